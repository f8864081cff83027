/*
 * wedlm_oracle.c -- CPU oracle for the WeDLM streaming-decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header, table or helper with
 * the HIP kernels.
 *
 * Plain C99 + OpenMP.  All arithmetic is float64.  The only roundings are at
 * the two storage points where the decode step stores a tensor in the model
 * dtype (the rotated queries and the rotated keys written to the cache);
 * there the value is rounded to that dtype (fp32 or bf16, nearest-even).
 * The one float decision of the method (the Eq. 11 threshold and its
 * fallback argmin) is taken in fp32, the precision of the GPU kernel, so
 * that both sides decide in the same precision; the fp64 margin of every
 * such decision is reported so tests can check it is far from float noise.
 *
 * Sources (the pages; cited by page title and section):
 *  [ABS]  "WeDLM: Reconciling Diffusion Language Models with Standard Causal
 *         Attention for Fast Inference", ICML 2026 oral page, abstract.
 *  [SUM]  Same title, paper-summary page (bud-325.pages.dev): "Key claims"
 *         (citing paper sec. 3.2, 4.1 Eq. 5-6, 5.2) and "Method" (training
 *         paragraph; inference paragraph with Eq. 11).
 *  [FEAT] risewithvishwas.com WeDLM page, "Core Technical Architecture"
 *         table and "Key Capabilities".
 *
 * Parity pins: every function below is checked by the CPU test suite
 * against closed forms, brute force on tiny inputs and invariants of the
 * method (tests/test_oracle_*.py); see the header comment of each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { WO_F32 = 0, WO_BF16 = 1, WO_F64 = 2 };

int wo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Storage rounding of a float64 value to fp32 or bf16 (nearest, ties to
 * even), or no rounding for float64 storage.  bf16 keeps 8 significant bits
 * and the fp32 exponent range.
 * ---------------------------------------------------------------------- */
double wo_round_storage(double x, int dtype) {
    if (dtype == WO_F64) return x;    /* float64 storage (toy-model checks) */
    if (dtype == WO_F32) return (double)(float)x;
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                     /* |x| = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                    /* quantum exponent for 8 significant bits */
    if (q < -133) q = -133;           /* bf16 subnormal quantum 2^-133 */
    double scaled = ldexp(x, -q);
    double r = nearbyint(scaled);     /* default rounding mode: ties to even */
    return ldexp(r, q);
}

/* ------------------------------------------------------------------------
 * Topological Reordering of one window ([SUM] Key claims, sec. 4.1 Eq. 5-6;
 * [SUM] Method, inference paragraph; [FEAT] "Architectural Bridging").
 * Observed (filled) slots move to the physical front, masked slots to the
 * back.  Inside each group the slots keep their slot order (the pages only
 * say observed-before-masked; keeping slot order is what makes the leading
 * committed run physically first and in order).
 * perm[r] = logical slot held by physical row r.  Returns the number of
 * observed slots.
 * ---------------------------------------------------------------------- */
int wo_reorder_perm(int W, const uint8_t *filled, int32_t *perm) {
    int r = 0;
    for (int i = 0; i < W; ++i)
        if (filled[i]) perm[r++] = i;
    int n_obs = r;
    for (int i = 0; i < W; ++i)
        if (!filled[i]) perm[r++] = i;
    return n_obs;
}

/* ------------------------------------------------------------------------
 * Rotary position embedding at a LOGICAL position p ([SUM] Key claims,
 * sec. 4.1: position ids keep the logical order; [FEAT] "Topological
 * Reordering": logical positions are carried by RoPE).  The pages do not
 * give the RoPE variant; the half-split pairing of the Qwen backbones is
 * used: coordinate c is paired with c + D/2 and rotated by the angle
 * p * base^(-2c/D).
 * ---------------------------------------------------------------------- */
void wo_rope(int D, double base, int32_t p, const double *x, double *y) {
    int h = D / 2;
    for (int c = 0; c < h; ++c) {
        double inv_freq = pow(base, -2.0 * (double)c / (double)D);
        double ang = (double)p * inv_freq;
        double cs = cos(ang), sn = sin(ang);
        double a = x[c], b = x[c + h];
        y[c] = a * cs - b * sn;
        y[c + h] = b * cs + a * sn;
    }
}

/* ------------------------------------------------------------------------
 * One reorder step for a batch: permutation, logical RoPE of queries and
 * keys, and the window's rows in physical order ready to be appended to the
 * prefix cache at positions L_b .. L_b+W-1 ([SUM] Method, inference
 * paragraph: the reordered window is run causally against the persistent
 * prefix cache).  Values are not rotated.
 *
 *   q [B][W][Hq][D], k/v [B][W][Hkv][D]  logical slot order, before RoPE
 *   q_phys [B][W][Hq][D]                 physical order, rotated, rounded
 *   k_win/v_win [B][W][Hkv][D]           physical order (k rotated, rounded)
 * Returns 0, or -1 if a row's positions are not strictly increasing.
 * ---------------------------------------------------------------------- */
int wo_reorder(int B, int W, int Hq, int Hkv, int D, int dtype, double base,
               const uint8_t *filled, const int32_t *pos,
               const double *q, const double *k, const double *v,
               int32_t *perm, double *q_phys, double *k_win, double *v_win) {
    for (int b = 0; b < B; ++b)
        for (int i = 1; i < W; ++i)
            if (pos[b * W + i] <= pos[b * W + i - 1]) return -1;
    for (int b = 0; b < B; ++b) {
        int32_t *pb = perm + (size_t)b * W;
        wo_reorder_perm(W, filled + (size_t)b * W, pb);
        for (int r = 0; r < W; ++r) {
            int slot = pb[r];
            int32_t p = pos[(size_t)b * W + slot];
            for (int h = 0; h < Hq; ++h) {
                const double *src = q + (((size_t)b * W + slot) * Hq + h) * D;
                double *dst = q_phys + (((size_t)b * W + r) * Hq + h) * D;
                wo_rope(D, base, p, src, dst);
                for (int d = 0; d < D; ++d) dst[d] = wo_round_storage(dst[d], dtype);
            }
            for (int g = 0; g < Hkv; ++g) {
                const double *ks = k + (((size_t)b * W + slot) * Hkv + g) * D;
                const double *vs = v + (((size_t)b * W + slot) * Hkv + g) * D;
                double *kd = k_win + (((size_t)b * W + r) * Hkv + g) * D;
                double *vd = v_win + (((size_t)b * W + r) * Hkv + g) * D;
                wo_rope(D, base, p, ks, kd);
                for (int d = 0; d < D; ++d) {
                    kd[d] = wo_round_storage(kd[d], dtype);
                    vd[d] = vs[d];
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Windowed causal attention of one decode step ([SUM] Key claims, sec. 3.2
 * and 5.2: a decode step attends the window rows causally over the cached
 * prefix and the earlier window rows; [FEAT] "Attention Mechanism": the
 * mask is the ordinary lower-triangular one).  Grouped-query attention: query head h reads KV head
 * h / (Hq/Hkv).
 *
 * For sequence b, query head h and physical row r the visible keys are the
 * L_b cached tokens plus window rows 0..r, i.e. dense key indices
 * 0 .. L_b + r.  o = sum_t softmax_t(scale * q.k_t) v_t, written at the
 * logical slot perm[r]:  out[b][perm[r]][h][:].
 *
 *   K/V   dense keys per sequence, [T_b][Hkv][D] at token offset kv_off[b]
 *         (T_b = L_b + W; the last W tokens are the appended window rows)
 *   rows  optional list of (b, r, h) triples; NULL computes every row
 * ---------------------------------------------------------------------- */
void wo_attention(int B, int W, int Hq, int Hkv, int D, double scale,
                  const double *q_phys, const double *K, const double *V,
                  const int64_t *kv_off, const int32_t *ctx_len,
                  const int32_t *perm, int64_t n_rows, const int32_t *rows,
                  double *out) {
    int G = Hq / Hkv;
    int64_t total = rows ? n_rows : (int64_t)B * W * Hq;
#pragma omp parallel
    {
        double *p = NULL;
        int64_t cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int64_t idx = 0; idx < total; ++idx) {
            int b, r, h;
            if (rows) {
                b = rows[3 * idx]; r = rows[3 * idx + 1]; h = rows[3 * idx + 2];
            } else {
                b = (int)(idx / ((int64_t)W * Hq));
                r = (int)((idx / Hq) % W);
                h = (int)(idx % Hq);
            }
            int g = h / G;
            int64_t nkeys = (int64_t)ctx_len[b] + r + 1;
            if (nkeys > cap) {
                free(p);
                cap = nkeys;
                p = (double *)malloc(sizeof(double) * (size_t)cap);
            }
            const double *qv = q_phys + (((size_t)b * W + r) * Hq + h) * D;
            double mx = -INFINITY;
            for (int64_t t = 0; t < nkeys; ++t) {
                const double *kv = K + ((size_t)(kv_off[b] + t) * Hkv + g) * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qv[d] * kv[d];
                p[t] = s * scale;
                if (p[t] > mx) mx = p[t];
            }
            double den = 0.0;
            for (int64_t t = 0; t < nkeys; ++t) {
                p[t] = exp(p[t] - mx);
                den += p[t];
            }
            double *o = out + (((size_t)b * W + perm[(size_t)b * W + r]) * Hq + h) * D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < nkeys; ++t) {
                const double *vv = V + ((size_t)(kv_off[b] + t) * Hkv + g) * D;
                double w = p[t] / den;
                for (int d = 0; d < D; ++d) o[d] += w * vv[d];
            }
        }
        free(p);
    }
}

/* ------------------------------------------------------------------------
 * Per-slot statistics of a logits row ([SUM] Method, inference paragraph:
 * the fill rule ranks masked slots by the entropy H_j of their predictive
 * distribution; the filled token is the most likely one).
 * argmax = lowest index of the maximum logit; H = Shannon entropy (nats) of
 * softmax(z) at temperature 1, evaluated as
 *     H = ln S - (1/S) * sum_v (z_v - m) e^{z_v - m},  S = sum_v e^{z_v - m}.
 * ---------------------------------------------------------------------- */
void wo_row_stats(int V, const float *z, int32_t *argmax, double *H) {
    double m = -INFINITY;
    int32_t a = 0;
    for (int i = 0; i < V; ++i)
        if ((double)z[i] > m) { m = (double)z[i]; a = i; }
    double S = 0.0, T = 0.0;
    for (int i = 0; i < V; ++i) {
        double u = (double)z[i] - m;
        double e = exp(u);
        S += e;
        T += u * e;
    }
    *argmax = a;
    *H = log(S) - T / S;
}

void wo_vocab_stats(int64_t R, int V, const float *logits, int32_t *argmax, double *H) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r)
        wo_row_stats(V, logits + (size_t)r * V, argmax + r, H + r);
}

/* ------------------------------------------------------------------------
 * Commit, select (Eq. 11) and refill for one streaming step ([SUM] Method,
 * inference paragraph; [SUM] Key claims, sec. 5.2; [ABS]: confident tokens
 * are committed into a growing left-to-right prefix).  Per sequence b:
 *
 *  1. commit: k = length of the leading run of filled slots; those tokens
 *     are emitted (committed[b][0..k) = tok, the rest -1), n_commit[b] = k
 *     and ctx_len[b] += k.  They were appended to the cache at L_b .. L_b+k-1
 *     by the reorder, so committing moves no data.
 *  2. select: over the masked slots j (all at j >= k), j0 = the leftmost
 *     one, d_j = j - j0, and the penalised entropy  Ht_j = H_j + alpha*d_j.
 *     Slots with Ht_j < tau are filled with their argmax token; if none
 *     passes, the single slot with the smallest Ht_j (lowest j on ties) is
 *     filled.  The decision is taken in fp32: Hf = (float)H,
 *     Ht = fmaf(alpha, (float)d, Hf), compared with (float)tau.
 *  3. refill: the window shifts left by k; k new masked slots (tok =
 *     mask_id) enter at the right; positions become ctx_len[b] + i.
 *
 * Rule readings (the pages give Eq. 11's form but not the fill rule): the
 * strict threshold, the at-least-one fallback and the tie-breaks are this
 * oracle's reading, shared by the GPU kernel.
 *
 * logits: rows of V fp32; row_index[b*W + j] is the row of slot (b, j) in
 * `logits` (-1 if not supplied; NULL = dense [B][W][V]).  Only masked slots
 * are read.  argmax_out / entropy_out [B][W] (may be NULL): masked slots get
 * their argmax and fp32 entropy, other slots -1 and -1.0f.
 * margin[b] (may be NULL): the smallest fp64 distance of any threshold
 * decision from tau, and, when the fallback ran, the gap between the two
 * smallest Ht values; +inf if no decision was taken.
 * Returns 0, or -1 if a masked slot's row was not supplied.
 * ---------------------------------------------------------------------- */
int wo_select_commit(int B, int W, int V, const float *logits, const int64_t *row_index,
                     int32_t *tok, uint8_t *filled, int32_t *pos, int32_t *ctx_len,
                     int32_t *n_commit, int32_t *committed,
                     int32_t *argmax_out, float *entropy_out,
                     double alpha, double tau, int32_t mask_id, double *margin) {
    int err = 0;
    for (int b = 0; b < B; ++b) {
        int32_t *tb = tok + (size_t)b * W;
        uint8_t *fb = filled + (size_t)b * W;
        /* 1. commit */
        int k = 0;
        while (k < W && fb[k]) ++k;
        n_commit[b] = k;
        for (int i = 0; i < W; ++i) committed[(size_t)b * W + i] = i < k ? tb[i] : -1;

        /* 2. select */
        int32_t *am = (int32_t *)malloc(sizeof(int32_t) * W);
        double *H = (double *)malloc(sizeof(double) * W);
        float *Hf = (float *)malloc(sizeof(float) * W);
        float *Ht = (float *)malloc(sizeof(float) * W);
        double *Ht64 = (double *)malloc(sizeof(double) * W);
        int j0 = -1;
        for (int j = 0; j < W; ++j) {
            am[j] = -1;
            Hf[j] = -1.0f;
            if (fb[j]) continue;
            if (j0 < 0) j0 = j;
            int64_t row = row_index ? row_index[(size_t)b * W + j] : (int64_t)b * W + j;
            if (row < 0) { err = -1; continue; }
            wo_row_stats(V, logits + (size_t)row * V, &am[j], &H[j]);
            Hf[j] = (float)H[j];
        }
        double mg = INFINITY;
        if (j0 >= 0) {
            const float a32 = (float)alpha, t32 = (float)tau;
            int any = 0;
            for (int j = j0; j < W; ++j) {
                if (fb[j]) continue;
                Ht[j] = fmaf(a32, (float)(j - j0), Hf[j]);
                Ht64[j] = H[j] + alpha * (double)(j - j0);
                double dm = fabs(Ht64[j] - tau);
                if (dm < mg) mg = dm;
                if (Ht[j] < t32) any = 1;
            }
            uint8_t *sel = (uint8_t *)calloc((size_t)W, 1);
            if (any) {
                for (int j = j0; j < W; ++j)
                    if (!fb[j] && Ht[j] < t32) sel[j] = 1;
            } else {
                int best = -1;
                for (int j = j0; j < W; ++j) {
                    if (fb[j]) continue;
                    if (best < 0 || Ht[j] < Ht[best]) best = j;
                }
                if (best < 0) best = j0; /* j0 is masked, so best is always set */
                sel[best] = 1;
                double gap = INFINITY;
                for (int j = j0; j < W; ++j)
                    if (!fb[j] && j != best) {
                        double gj = fabs(Ht64[j] - Ht64[best]);
                        if (gj < gap) gap = gj;
                    }
                if (gap < mg) mg = gap;
            }
            for (int j = 0; j < W; ++j)
                if (sel[j]) { tb[j] = am[j]; fb[j] = 1; }
            free(sel);
        }
        if (margin) margin[b] = mg;
        if (argmax_out)
            for (int j = 0; j < W; ++j) argmax_out[(size_t)b * W + j] = am[j];
        if (entropy_out)
            for (int j = 0; j < W; ++j) entropy_out[(size_t)b * W + j] = Hf[j];

        /* 3. refill */
        for (int i = 0; i < W; ++i) {
            if (i + k < W) { tb[i] = tb[i + k]; fb[i] = fb[i + k]; }
            else { tb[i] = mask_id; fb[i] = 0; }
        }
        ctx_len[b] += k;
        for (int i = 0; i < W; ++i) pos[(size_t)b * W + i] = ctx_len[b] + i;
        free(am); free(H); free(Hf); free(Ht); free(Ht64);
    }
    return err;
}
