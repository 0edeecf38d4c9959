/*
 * any4 quantizer: CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the HIP
 * library under weight_only_bit_row_amd/) shares no code, header, table or
 * constant with this file.
 *
 * Plain, single-threaded, slow on purpose: every step is written out the way
 * "any4: Learned 4-bit Numeric Representation for LLMs" (arXiv 2507.04610) states
 * it, so that a reader can check it against the paper by eye.  Build with
 * -O2 -ffp-contract=off so that no multiply-add is fused.
 *
 * Precision: the scaled weights (Section 2.5.1, Eq. 1-2), the sample weights,
 * the squared distances of the E-step (Section 4.1, Eq. 18) and the k-means++
 * sampling weights are fp32, because they decide integers (codes, picks) and
 * both sides must take those decisions in the same precision.  The M-step sums
 * (Eq. 23) and the objective are fp64.
 *
 * Pinned by tests/test_oracle_*.py (closed forms, brute-force / DP optimum,
 * scikit-learn Lloyd, numpy Philox4x64, numpy float16 casts, the storage cost
 * printed in Section 2.4.1; for the bookends E|x| and Eq. 4 dequantization, exact
 * rational means, a worked example, exact reconstruction of exact-level rows and
 * torch's bfloat16 cast; for the method variants, exact invariances, nearest-level
 * codes, draw frequencies and restart minima).  Philox4x32-10 is pinned against
 * rocRAND's implementation of the same generator (its host-callable engine).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_INVALID_ARG 1
#define ORACLE_ERR_NONFINITE 5

/* Sample weights above this bound are rejected together with non-finite values, so
 * that fp32 sums over a row can never overflow (2^64 * 15 * 2^22 < 2^128). */
#define ORACLE_A_MAX 18446744073709551616.0f /* 2^64 */

int oracle_any4_version(void) { return 1; }

/* ------------------------------------------------------------------------- */
/* Philox-4xW-10, from Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
 * as easy as 1, 2, 3" (SC'11), Section 4.  One round multiplies words 0 and 2 by
 * the two round multipliers, then forms the new 4-word state from the products'
 * high halves xor-ed with the other two words and the round key, and from the
 * products' low halves.  The key is bumped by the two Weyl constants between
 * rounds.  The 64-bit variant (checked against numpy.random.Philox) and the
 * 32-bit variant (checked against rocRAND's engine) share this structure through one
 * macro. */

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

static inline void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

#define PHILOX4_ROUNDS(T, MULHILO, M0, M1, W0, W1, ctr, key, out)            \
    do {                                                                     \
        T x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];                \
        T k0 = key[0], k1 = key[1];                                          \
        for (int round = 0; round < 10; ++round) {                           \
            if (round > 0) { k0 += (T)(W0); k1 += (T)(W1); }                 \
            T hi0, lo0, hi1, lo1;                                            \
            MULHILO((T)(M0), x0, &hi0, &lo0);                                \
            MULHILO((T)(M1), x2, &hi1, &lo1);                                \
            T y0 = hi1 ^ x1 ^ k0;                                            \
            T y1 = lo1;                                                      \
            T y2 = hi0 ^ x3 ^ k1;                                            \
            T y3 = lo0;                                                      \
            x0 = y0; x1 = y1; x2 = y2; x3 = y3;                              \
        }                                                                    \
        out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;                  \
    } while (0)

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    PHILOX4_ROUNDS(uint32_t, mulhilo32, 0xD2511F53u, 0xCD9E8D57u, 0x9E3779B9u, 0xBB67AE85u,
                   ctr, key, out);
}

void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
    PHILOX4_ROUNDS(uint64_t, mulhilo64, 0xD2E7470EE14C6C93ull, 0xCA5A826395121157ull,
                   0x9E3779B97F4A7C15ull, 0xBB67AE8584CAA73Bull, ctr, key, out);
}

/* ------------------------------------------------------------------------- */
/* IEEE binary16 with round-to-nearest-even, from the binary32 bit pattern.
 * The LUT is stored as 16 fp16 values and each group as two fp16 values
 * (OpenReview rebuttal; Section 2.4.1 of the paper). */
static uint16_t fp16_rne(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t e = (x >> 23) & 0xFFu;
    uint32_t m = x & 0x7FFFFFu;
    if (e == 0xFFu) {                       /* inf or nan */
        if (m == 0) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u | (m >> 13));
    }
    int32_t exp = (int32_t)e - 127;         /* unbiased */
    if (exp > 15) return (uint16_t)(sign | 0x7C00u);   /* overflow: > 65504 range */
    if (exp >= -14) {                       /* normal fp16 range */
        uint32_t mant = m;                  /* 23 bits, keep 10 */
        uint32_t keep = mant >> 13;
        uint32_t rest = mant & 0x1FFFu;
        uint32_t h = ((uint32_t)(exp + 15) << 10) | keep;
        if (rest > 0x1000u || (rest == 0x1000u && (keep & 1u))) h += 1;  /* may carry into exp */
        return (uint16_t)(sign | h);        /* carry into 0x7C00 gives inf, as it should */
    }
    /* subnormal fp16 (or underflow to zero): value = mant24 * 2^(exp-23),
     * fp16 subnormal unit is 2^-24, so the count is mant24 * 2^(exp-23+24). */
    if (e == 0) return (uint16_t)sign;      /* fp32 zero or subnormal: far below 2^-25 */
    uint32_t mant24 = m | 0x800000u;
    int32_t shift = -(exp + 1);             /* right shift so that unit = 2^-24 */
    /* exp in [-127+1, -15]: shift in [14, 126] */
    if (shift > 24 + 1) return (uint16_t)sign;
    uint32_t keep = mant24 >> shift;
    uint32_t rest = mant24 & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rest > half || (rest == half && (keep & 1u))) keep += 1;
    return (uint16_t)(sign | keep);         /* keep == 0x400 becomes the smallest normal */
}

uint16_t oracle_fp16_rne(float f) { return fp16_rne(f); }

void oracle_fp16_rne_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = fp16_rne(in[i]);
}

static float bf16_to_f32(uint16_t b) {
    uint32_t x = (uint32_t)b << 16;
    float f;
    memcpy(&f, &x, 4);
    return f;
}

/* ------------------------------------------------------------------------- */
/* Step 1: group-wise asymmetric min/max scaling, Section 2.5.1 Eq. 1 and Eq. 2.
 * Groups are g contiguous elements of the row, t*g <= j < (t+1)*g (the paper
 * prints the range as kg <= j < k(g+1); the corrected range is used).
 * alpha = (max - min) / (Qmax - Qmin) with Qmax - Qmin = 2^n - 1, beta = min,
 * w_S = (w - beta) / alpha.  A constant group (alpha = 0) gets w_S = 0.
 * Returns 0, or 1 when a value or alpha is not finite. */
int oracle_scale_row_mode(const float* w, int64_t K, int32_t group, int32_t qr, int32_t symmetric,
                          float* ws, float* alpha, float* beta) {
    int bad = 0;
    for (int64_t t = 0; t < K / group; ++t) {
        const float* wg = w + t * group;
        float mn = wg[0], mx = wg[0], amax = 0.0f;
        for (int64_t j = 0; j < group; ++j) {
            if (!isfinite(wg[j])) bad = 1;
            if (wg[j] < mn) mn = wg[j];
            if (wg[j] > mx) mx = wg[j];
            if (fabsf(wg[j]) > amax) amax = fabsf(wg[j]);
        }
        float al, be;
        if (symmetric) {
            /* Eq. 3: alpha = max|w| / Qmax, beta = 0, with Qmax = 2^(n-1) (the int4 span
             * -7..+8 of Section 2.5.1 has Qmax = 8), so w_S lies in [-Qmax, Qmax] */
            al = amax / (float)((qr + 1) / 2);
            be = 0.0f;
        } else {
            float range = mx - mn;
            al = range / (float)qr;
            be = mn;
        }
        if (!isfinite(al)) bad = 1;
        alpha[t] = al;
        beta[t] = be;
        mn = be;
        for (int64_t j = 0; j < group; ++j) {
            if (al > 0.0f) {
                float diff = wg[j] - mn;
                ws[t * group + j] = diff / al;
            } else {
                ws[t * group + j] = 0.0f;
            }
        }
    }
    return bad;
}

int oracle_scale_row(const float* w, int64_t K, int32_t group, int32_t qr,
                     float* ws, float* alpha, float* beta) {
    return oracle_scale_row_mode(w, K, group, qr, 0, ws, alpha, beta);
}

/* Step 2: the per-element sample weight of Eq. 23, alpha_{i,j} * E|x_j|, in fp32.
 * Returns 1 when an activation statistic is negative or not finite, or a weight
 * is not finite or above the bound. */
int oracle_weights_row_mode(const float* alpha, const float* act, int64_t K, int32_t group,
                            int32_t weighting, float* a) {
    int bad = 0;
    for (int64_t j = 0; j < K; ++j) {
        if (!isfinite(act[j]) || act[j] < 0.0f) bad = 1;
        if (weighting == 0)
            a[j] = alpha[j / group] * act[j];
        else if (weighting == 1)
            a[j] = act[j];
        else
            a[j] = 1.0f;
        if (!isfinite(a[j]) || a[j] > ORACLE_A_MAX) bad = 1;
    }
    return bad;
}

/* The minimization terms of Appendix C.1 (Table A3): weighting 0 is Eq. 23's
 * alpha * E|x| (the default), 1 uses E|x| alone, 2 the plain scaled weights (a = 1). */
int oracle_weights_row(const float* alpha, const float* act, int64_t K, int32_t group, float* a) {
    return oracle_weights_row_mode(alpha, act, K, group, 0, a);
}

static float sqdist(float x, float c) {
    float d = x - c;
    return d * d;
}

/* Step 3: weighted k-means++ seeding (D^2 sampling, Arthur and Vassilvitskii 2007,
 * which the paper's Appendix C.2 names as scikit-learn's default init).  The
 * first centre is drawn with probability proportional to the sample weight a_j,
 * every later one proportional to a_j * D_j, where D_j is the squared distance to
 * the nearest centre drawn so far.
 *
 * Sampling is done exactly in integers, with a fixed-point scale 2^(40-e):
 * q_j = floor(p_j * 2^(40-e)), Q = sum q_j, and one Philox4x32-10 draw per (row, t):
 * u = x1 * 2^32 + x0 with counter (lo32(row), t, matrix, hi32(row)) and key
 * (lo32(seed), hi32(seed)); r = floor(u * Q / 2^64); the pick is the smallest j whose
 * prefix sum of q exceeds r.  e = floor(log2 B) for a bound B on the draw's weights:
 * B = max_j a_j for the first draw; for every later draw one bound, set after the first
 * pick: B = fl(max_j a_j * fl(m * m)) with m = max(fl(x_max - c_0), fl(c_0 - x_min))
 * over the row's scaled weights, which no later weight a_j * D_j exceeds (D_j only
 * decreases, and rounding is monotone), so every q_j stays below 2^41.  (For the random
 * initialization, whose weights are the a_j of the elements not yet drawn, B = max_j a_j
 * throughout.)  When B = 0 or Q = 0 (every weight is 0, or below 2^(e-40)) the centre is
 * copied from w_S[0] (t = 0) or from centre 0 (t > 0) and its pick is -1.
 * From the second draw on (k-means++ and greedy), when s = 40 - e >= 0 the sample weight
 * is scaled by the power of two before the product instead of after it:
 * p_j = fl(fl(a_j * 2^s) * D_j) and q_j = floor(p_j).  fl(a_j * 2^s) is exact, so this
 * equals floor(fl(a_j * D_j) * 2^s) whenever a_j * D_j is a normal fp32 number; the two
 * differ only for products below 2^-126 in rows whose bound is below 2^-86. */
/* Initial centres for the initializations of Appendix C.2 (Table A4):
 *   init 0  k-means++ as described above;
 *   init 1  random: k distinct elements drawn one after another, each with probability
 *           proportional to a_j among the elements not yet drawn (scikit-learn's random
 *           init with sample weights), with the same integer sampling and Philox draws;
 *   init 2  uniform: the integer levels, c_t = level0 + t (int4's -7..8 up to the
 *           translation of the scaled domain: level0 = 0 for asymmetric scaling,
 *           1 - k/2 for symmetric); no draws, picks = -1.
 *   init 3  greedy k-means++ (the variant scikit-learn runs by default): the first centre
 *           as in k-means++; each later draw takes L = 2 + floor(ln k) candidates from
 *           the same D^2 distribution (candidate s from Philox counter word
 *           t + 16 * restart + 65536 * s, so candidate 0 is the plain draw) and keeps the
 *           one whose potential, sum_j floor(a_j * min(D_j, (w_S_j - c)^2) * 2^(40-e))
 *           with e of this draw (the weight scaled before the product, as above), is
 *           smallest (the lowest s on equal potentials).  The
 *           potentials are integers, so they compare exactly.
 * `restart` selects an independent draw stream for restarts: the Philox counter's
 * second word is t + 16 * restart. */

/* Candidates per greedy draw: 2 + floor(ln k) for k = 2, 4, 8, 16. */
int32_t oracle_greedy_trials(int32_t k) {
    return 2 + (int32_t)floor(log((double)k));
}

/* The index whose prefix sum of q first exceeds r (the last index if none does). */
static int64_t first_crossing(const uint64_t* q, int64_t K, uint64_t r) {
    uint64_t prefix = 0;
    for (int64_t j = 0; j < K; ++j) {
        prefix += q[j];
        if (prefix > r) return j;
    }
    return K - 1;
}

static uint64_t philox_u64(uint64_t seed, uint64_t row_id, uint32_t word1, uint32_t matrix_index) {
    uint32_t ctr[4] = {(uint32_t)row_id, word1, matrix_index, (uint32_t)(row_id >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    oracle_philox4x32_10(ctr, key, x);
    return ((uint64_t)x[1] << 32) | (uint64_t)x[0];
}

int oracle_seed_row_init(const float* ws, const float* a, int64_t K, int32_t k,
                         uint64_t seed, uint64_t row_id, uint32_t matrix_index,
                         int32_t init, int32_t restart, float level0,
                         float* c0, int32_t* picks) {
    if (init == 2) {
        for (int32_t t = 0; t < k; ++t) {
            c0[t] = level0 + (float)t;
            picks[t] = -1;
        }
        return ORACLE_OK;
    }
    float* D = (float*)malloc((size_t)K * sizeof(float));
    float* p = (float*)malloc((size_t)K * sizeof(float));
    uint64_t* q = (uint64_t*)malloc((size_t)K * sizeof(uint64_t));
    if (!D || !p || !q) { free(D); free(p); free(q); return ORACLE_ERR_INVALID_ARG; }

    /* bound of the first draw's weights, and the row's extremes for the later bound */
    float a_max = 0.0f, x_min = ws[0], x_max = ws[0];
    for (int64_t j = 0; j < K; ++j) {
        if (a[j] > a_max) a_max = a[j];
        if (ws[j] < x_min) x_min = ws[j];
        if (ws[j] > x_max) x_max = ws[j];
    }
    float B = a_max;
    for (int32_t t = 0; t < k; ++t) {
        if (t == 1 && init != 1) {
            const float up = x_max - c0[0], down = c0[0] - x_min;
            const float m = up > down ? up : down;
            B = a_max * (m * m);
        }
        int e = 0;
        if (B > 0.0f) {
            int E;
            frexp((double)B, &E);               /* B = f * 2^E, f in [0.5, 1) */
            e = E - 1;                           /* floor(log2 B) */
        }
        /* the weights scaled by 2^s before the product (see above) */
        const int prescaled = (t > 0 && init != 1 && 40 - e >= 0);
        for (int64_t j = 0; j < K; ++j) {
            if (init == 1)
                p[j] = (t == 0) ? a[j] : p[j];    /* drawn elements were set to 0 below */
            else if (t == 0)
                p[j] = a[j];
            else if (prescaled)
                p[j] = ldexpf(a[j], 40 - e) * D[j];
            else
                p[j] = a[j] * D[j];
        }
        uint64_t Q = 0;
        if (B > 0.0f) {
            for (int64_t j = 0; j < K; ++j) {
                double v = prescaled ? (double)p[j] : ldexp((double)p[j], 40 - e);
                q[j] = (uint64_t)floor(v);
                Q += q[j];
            }
        }
        if (Q == 0) {
            c0[t] = (t == 0) ? ws[0] : c0[0];
            picks[t] = -1;
        } else {
            const uint32_t word1 = (uint32_t)(t + 16 * restart);
            uint64_t u = philox_u64(seed, row_id, word1, matrix_index);
            uint64_t r = (uint64_t)(((unsigned __int128)u * (unsigned __int128)Q) >> 64);
            int64_t pick = first_crossing(q, K, r);
            if (init == 3 && t > 0) {
                /* greedy: more candidates, keep the one with the smallest potential */
                const double sc = ldexp(1.0, 40 - e);
                uint64_t best_pot = 0;
                for (int32_t s = 0; s < oracle_greedy_trials(k); ++s) {
                    int64_t cand = pick;
                    if (s > 0) {
                        uint64_t us = philox_u64(seed, row_id, word1 + 65536u * (uint32_t)s,
                                                 matrix_index);
                        uint64_t rs = (uint64_t)(((unsigned __int128)us * (unsigned __int128)Q) >> 64);
                        cand = first_crossing(q, K, rs);
                    }
                    uint64_t pot = 0;
                    for (int64_t j = 0; j < K; ++j) {
                        float d = sqdist(ws[j], ws[cand]);
                        float m = d < D[j] ? d : D[j];
                        pot += prescaled ? (uint64_t)floor((double)(ldexpf(a[j], 40 - e) * m))
                                         : (uint64_t)floor((double)(a[j] * m) * sc);
                    }
                    if (s == 0 || pot < best_pot) {
                        best_pot = pot;
                        if (s > 0) pick = cand;
                    }
                }
            }
            c0[t] = ws[pick];
            picks[t] = (int32_t)pick;
            if (init == 1) p[pick] = 0.0f;
        }
        if (init != 1) {
            for (int64_t j = 0; j < K; ++j) {
                float d = sqdist(ws[j], c0[t]);
                if (t == 0 || d < D[j]) D[j] = d;
            }
        }
    }
    free(D); free(p); free(q);
    return ORACLE_OK;
}

int oracle_seed_row(const float* ws, const float* a, int64_t K, int32_t k,
                    uint64_t seed, uint64_t row_id, uint32_t matrix_index,
                    float* c0, int32_t* picks) {
    return oracle_seed_row_init(ws, a, K, k, seed, row_id, matrix_index, 0, 0, 0.0f, c0, picks);
}

/* Step 4a: E-step, Section 4.1 Eq. 18: each scaled weight goes to the LUT value
 * with the smallest squared distance; on equal distances the lowest index wins. */
void oracle_estep_row(const float* ws, int64_t K, const float* c, int32_t k, uint8_t* q) {
    for (int64_t j = 0; j < K; ++j) {
        int best = 0;
        float bd = sqdist(ws[j], c[0]);
        for (int t = 1; t < k; ++t) {
            float d = sqdist(ws[j], c[t]);
            if (d < bd) { bd = d; best = t; }
        }
        q[j] = (uint8_t)best;
    }
}

/* Step 4b: M-step, Section 4.1 Eq. 23: each LUT value becomes the mean of its
 * cluster's scaled weights weighted by alpha_{i,j} * E|x_j|.  A cluster whose
 * weight sum is 0 keeps its previous value. */
void oracle_mstep_row(const float* ws, const float* a, const uint8_t* q, int64_t K,
                      const float* c_prev, int32_t k, float* c_new) {
    double S1[16], S0[16];
    for (int t = 0; t < k; ++t) { S1[t] = 0.0; S0[t] = 0.0; }
    for (int64_t j = 0; j < K; ++j) {
        S1[q[j]] += (double)a[j] * (double)ws[j];
        S0[q[j]] += (double)a[j];
    }
    for (int t = 0; t < k; ++t)
        c_new[t] = (S0[t] > 0.0) ? (float)(S1[t] / S0[t]) : c_prev[t];
}

/* The weighted objective that the E/M alternation decreases:
 * J = sum_j a_j (w_S_j - c_{q_j})^2, in fp64. */
double oracle_objective_row(const float* ws, const float* a, const uint8_t* q, int64_t K,
                            const float* c) {
    double J = 0.0;
    for (int64_t j = 0; j < K; ++j) {
        double d = (double)ws[j] - (double)c[q[j]];
        J += (double)a[j] * d * d;
    }
    return J;
}

/* Step 6: codes, two per byte, the even column in the low nibble. */
void oracle_pack_row(const uint8_t* q, int64_t K, uint8_t* codes) {
    for (int64_t m = 0; m < K / 2; ++m)
        codes[m] = (uint8_t)((q[2 * m] & 0xF) | ((q[2 * m + 1] & 0xF) << 4));
}

/* ------------------------------------------------------------------------- */
/* The whole path for rows [0, n_rows) of one matrix, row-major.
 * Per row (Algorithm 1 of the paper's Appendix A, minus the calibration and the
 * module loop): scale, weights, initial centres, `iters` rounds of E-step then
 * M-step, a final E-step, then emission (fp16 LUT in draw order, fp16 alpha and
 * beta, nibble-packed codes).
 *
 * `variant` selects the method variants of the paper's ablations (0 = the defaults):
 *   bits 0-1   sample weights (Appendix C.1): 0 alpha*E|x|, 1 E|x|, 2 none (a = 1)
 *   bits 2-3   initialization (Appendix C.2): 0 k-means++, 1 random, 2 uniform levels
 *   bit 4      symmetric scaling (Eq. 3) instead of asymmetric (Eq. 2)
 *   bits 8-15  restarts - 1: the whole k-means runs from that many initializations
 *              (Philox streams t + 16 r) and the one with the lowest final objective
 *              is kept (the earliest on ties), as scikit-learn's n_init does
 * Any other bit set, or a field value not listed, is an invalid argument.
 *
 * Traces are optional (NULL to skip) and belong to the restart that is kept:
 *   c_trace [n_rows, iters+1, k]  centroids c^0 .. c^iters
 *   j_trace [n_rows, iters+1]     J at c^0 .. c^iters, each with the E-step
 *                                 assignment at those centroids
 *   picks   [n_rows, k]           initial picks (-1 where no element was drawn)
 *   c_final [n_rows, k]           fp32 centroids before the fp16 cast
 * A row with a non-finite input, a negative activation statistic, a non-finite
 * alpha or a too-large weight gets zero outputs and a NaN objective, and the call
 * returns ORACLE_ERR_NONFINITE after finishing the other rows. */
int oracle_any4_quantize_v(const void* w, int32_t dtype, int64_t n_rows, int64_t n_cols,
                           const float* act, int64_t row_offset, int32_t matrix_index,
                           int32_t group, int32_t n_clusters, int32_t iters, uint64_t seed,
                           int32_t variant,
                           uint8_t* codes, uint16_t* lut, uint16_t* scale, uint16_t* offset,
                           double* objective, float* c_trace, double* j_trace,
                           int32_t* picks, float* c_final) {
    const int64_t K = n_cols;
    const int32_t k = n_clusters;
    const int32_t weighting = variant & 3, init = (variant >> 2) & 3, symmetric = (variant >> 4) & 1;
    const int32_t restarts = ((variant >> 8) & 0xFF) + 1;
    if (n_rows < 0 || K < 2 || (K & 1) || group < 1 || K % group != 0 || iters < 0 ||
        (dtype != 0 && dtype != 1) || row_offset < 0 ||
        !(k == 2 || k == 4 || k == 8 || k == 16) || weighting == 3 ||
        (variant & ~0xFF1F) != 0)
        return ORACLE_ERR_INVALID_ARG;
    const int32_t qr = k - 1;
    const float level0 = symmetric ? (float)(1 - k / 2) : 0.0f;
    const int64_t G = K / group;
    float* wrow = (float*)malloc((size_t)K * sizeof(float));
    float* ws = (float*)malloc((size_t)K * sizeof(float));
    float* a = (float*)malloc((size_t)K * sizeof(float));
    float* alpha = (float*)malloc((size_t)G * sizeof(float));
    float* beta = (float*)malloc((size_t)G * sizeof(float));
    uint8_t* q = (uint8_t*)malloc((size_t)K);
    float* ct = (float*)malloc((size_t)(iters + 1) * 16 * sizeof(float));
    double* jt = (double*)malloc((size_t)(iters + 1) * sizeof(double));
    if (!wrow || !ws || !a || !alpha || !beta || !q || !ct || !jt) {
        free(wrow); free(ws); free(a); free(alpha); free(beta); free(q); free(ct); free(jt);
        return ORACLE_ERR_INVALID_ARG;
    }
    int status = ORACLE_OK;
    for (int64_t i = 0; i < n_rows; ++i) {
        if (dtype == 0) {
            memcpy(wrow, (const float*)w + i * K, (size_t)K * sizeof(float));
        } else {
            const uint16_t* wb = (const uint16_t*)w + i * K;
            for (int64_t j = 0; j < K; ++j) wrow[j] = bf16_to_f32(wb[j]);
        }
        int bad = oracle_scale_row_mode(wrow, K, group, qr, symmetric, ws, alpha, beta);
        bad |= oracle_weights_row_mode(alpha, act, K, group, weighting, a);
        for (int64_t j = 0; j < K && !bad; ++j)
            if (!isfinite(a[j] * ws[j])) bad = 1;
        if (bad) {
            status = ORACLE_ERR_NONFINITE;
            memset(codes + i * (K / 2), 0, (size_t)(K / 2));
            memset(lut + i * k, 0, (size_t)k * 2);
            memset(scale + i * G, 0, (size_t)G * 2);
            memset(offset + i * G, 0, (size_t)G * 2);
            if (objective) objective[i] = NAN;
            continue;
        }
        float best_c[16];
        double best_j = INFINITY;
        for (int32_t r = 0; r < restarts; ++r) {
            float c[16], cn[16];
            int32_t pk[16];
            oracle_seed_row_init(ws, a, K, k, seed, (uint64_t)(row_offset + i),
                                 (uint32_t)matrix_index, init, r, level0, c, pk);
            double J = 0.0;
            for (int32_t it = 0; it <= iters; ++it) {
                oracle_estep_row(ws, K, c, k, q);
                memcpy(ct + (size_t)it * k, c, (size_t)k * sizeof(float));
                jt[it] = oracle_objective_row(ws, a, q, K, c);
                if (it == iters) { J = jt[it]; break; }
                oracle_mstep_row(ws, a, q, K, c, k, cn);
                memcpy(c, cn, sizeof(c));
            }
            if (r == 0 || J < best_j) {      /* the earliest restart wins ties */
                best_j = J;
                memcpy(best_c, c, sizeof(best_c));
                if (picks) memcpy(picks + i * k, pk, (size_t)k * sizeof(int32_t));
                if (c_trace) memcpy(c_trace + i * (iters + 1) * k, ct, (size_t)(iters + 1) * k * sizeof(float));
                if (j_trace) memcpy(j_trace + i * (iters + 1), jt, (size_t)(iters + 1) * sizeof(double));
            }
        }
        /* final E-step at the kept centroids */
        oracle_estep_row(ws, K, best_c, k, q);
        if (objective) objective[i] = oracle_objective_row(ws, a, q, K, best_c);
        if (c_final) memcpy(c_final + i * k, best_c, (size_t)k * sizeof(float));
        oracle_pack_row(q, K, codes + i * (K / 2));
        for (int t = 0; t < k; ++t) lut[i * k + t] = fp16_rne(best_c[t]);
        for (int64_t g = 0; g < G; ++g) {
            scale[i * G + g] = fp16_rne(alpha[g]);
            offset[i * G + g] = fp16_rne(beta[g]);
        }
    }
    free(wrow); free(ws); free(a); free(alpha); free(beta); free(q); free(ct); free(jt);
    return status;
}

int oracle_any4_quantize(const void* w, int32_t dtype, int64_t n_rows, int64_t n_cols,
                         const float* act, int64_t row_offset, int32_t matrix_index,
                         int32_t group, int32_t n_clusters, int32_t iters, uint64_t seed,
                         uint8_t* codes, uint16_t* lut, uint16_t* scale, uint16_t* offset,
                         double* objective, float* c_trace, double* j_trace,
                         int32_t* picks, float* c_final) {
    return oracle_any4_quantize_v(w, dtype, n_rows, n_cols, act, row_offset, matrix_index, group,
                                  n_clusters, iters, seed, 0, codes, lut, scale, offset, objective,
                                  c_trace, j_trace, picks, c_final);
}

/* ------------------------------------------------------------------------- */
/* Bookends of the quantizer: the calibration statistic it consumes and the
 * dequantization of what it emits. */

/* IEEE binary16 bit pattern to binary32 (exact: every fp16 value is an fp32 value).
 * Sign, 5-bit exponent with bias 15, 10-bit fraction; exponent 0 holds zero and the
 * subnormals (fraction * 2^-24), exponent 31 holds inf and NaN. */
static float fp16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1Fu;
    const uint32_t f = h & 0x3FFu;
    float mag;
    if (e == 0) {
        mag = (float)f * 0x1p-24f;                       /* zero or subnormal, exact */
    } else if (e == 0x1F) {
        uint32_t x = 0x7F800000u | (f << 13);            /* inf, or NaN keeping its payload */
        memcpy(&mag, &x, 4);
    } else {
        uint32_t x = ((e - 15 + 127) << 23) | (f << 13);  /* normal: rebias the exponent */
        memcpy(&mag, &x, 4);
    }
    uint32_t bits;
    memcpy(&bits, &mag, 4);
    bits |= sign;
    float out;
    memcpy(&out, &bits, 4);
    return out;
}

float oracle_fp16_to_f32(uint16_t h) { return fp16_to_f32(h); }

/* binary32 to bfloat16 (the upper 16 bits) with round-to-nearest-even on the
 * discarded 16 bits; NaN stays a quiet NaN. */
static uint16_t bf16_rne(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    if ((x & 0x7F800000u) == 0x7F800000u && (x & 0x7FFFFFu)) return (uint16_t)((x >> 16) | 0x40u);
    const uint32_t keep = x >> 16, rest = x & 0xFFFFu;
    uint32_t r = keep;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) r += 1;   /* may carry to inf */
    return (uint16_t)r;
}

void oracle_bf16_rne_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(in[i]);
}

/* E|x_j| of Section 4.1: the mean over the calibration tokens of the absolute
 * activation of input channel j.  x is [T, K] row-major (token t, channel j), fp32
 * (dtype 0) or bf16 bits (dtype 1).  Each channel's |x| values are summed in fp64
 * in token order, the sum is divided by T in fp64 and rounded to fp32.
 * Returns 1 for T < 1 or K < 1. */
int oracle_act_absmean(const void* x, int32_t dtype, int64_t T, int64_t K, float* out) {
    if (T < 1 || K < 1 || (dtype != 0 && dtype != 1)) return ORACLE_ERR_INVALID_ARG;
    for (int64_t j = 0; j < K; ++j) {
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const float v = dtype == 0 ? ((const float*)x)[t * K + j]
                                       : bf16_to_f32(((const uint16_t*)x)[t * K + j]);
            s += fabs((double)v);
        }
        out[j] = (float)(s / (double)T);
    }
    return ORACLE_OK;
}

/* Dequantization, Section 2.5.2 (Eq. 4): dequant(w_Q) = alpha * w_Q + beta, where for
 * any4 the rounded value w_Q of element (i, j) is the row's LUT entry at its code.
 * The fp16 LUT, scale (alpha) and offset (beta) are widened to fp32 and the value is
 * fl(fl(alpha * LUT[q]) + beta) in fp32, product and sum rounded separately.
 * codes [N, K/2] (byte m: column 2m in the low nibble), lut [N, k], scale and
 * offset [N, K/group]; out [N, K] fp32. */
int oracle_dequantize(const uint8_t* codes, const uint16_t* lut, const uint16_t* scale,
                      const uint16_t* offset, int64_t N, int64_t K, int32_t group,
                      int32_t k, float* out) {
    if (N < 0 || K < 2 || (K & 1) || group < 1 || K % group != 0 || k < 1 || k > 16)
        return ORACLE_ERR_INVALID_ARG;
    const int64_t G = K / group;
    for (int64_t i = 0; i < N; ++i) {
        for (int64_t j = 0; j < K; ++j) {
            const uint8_t byte = codes[i * (K / 2) + j / 2];
            const int q = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            const float level = q < k ? fp16_to_f32(lut[i * k + q]) : NAN;
            const float alpha = fp16_to_f32(scale[i * G + j / group]);
            const float beta = fp16_to_f32(offset[i * G + j / group]);
            const float prod = alpha * level;
            out[i * K + j] = prod + beta;
        }
    }
    return ORACLE_OK;
}

/* LUT-dequantized matrix-vector products (the inference consumer of the emitted
 * format; the paper's tinygemm kernels dequantize weights on the fly before the
 * multiply, Section 4.2): y[m, i] = sum_j x[m, j] * w_hat[i, j], with w_hat the Eq. 4
 * dequantization above (fp32) and x [M, K] fp32 or bf16 bits (dtype); each product is
 * exact in fp64 and the sum runs in fp64 in column order; y [M, N] is that sum rounded
 * to fp32.  Also returns, per output, the magnitude scale
 * s[m, i] = sum_j |x[m, j]| * (|fl(alpha * LUT[q])| + |beta|) in fp64, against which a
 * differently ordered fp32 evaluation is judged. */
int oracle_lut_gemv(const uint8_t* codes, const uint16_t* lut, const uint16_t* scale,
                    const uint16_t* offset, int64_t N, int64_t K, int32_t group, int32_t k,
                    const void* x, int32_t dtype, int64_t M, float* y, double* s) {
    if (M < 1 || N < 0 || K < 2 || (K & 1) || group < 1 || K % group != 0 || k < 1 || k > 16 ||
        (dtype != 0 && dtype != 1))
        return ORACLE_ERR_INVALID_ARG;
    const int64_t G = K / group;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t i = 0; i < N; ++i) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                const uint8_t byte = codes[i * (K / 2) + j / 2];
                const int q = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                const float level = q < k ? fp16_to_f32(lut[i * k + q]) : NAN;
                const float alpha = fp16_to_f32(scale[i * G + j / group]);
                const float beta = fp16_to_f32(offset[i * G + j / group]);
                const float prod = alpha * level;
                const float w = prod + beta;
                const float xv = dtype == 0 ? ((const float*)x)[m * K + j]
                                            : bf16_to_f32(((const uint16_t*)x)[m * K + j]);
                acc += (double)xv * (double)w;
                mag += fabs((double)xv) * (fabs((double)prod) + fabs((double)beta));
            }
            y[m * N + i] = (float)acc;
            if (s) s[m * N + i] = mag;
        }
    }
    return ORACLE_OK;
}
