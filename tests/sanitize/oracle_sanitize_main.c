/* Host sanitizer driver for the CPU oracle (test infrastructure).
 *
 * Built with gcc -fsanitize=address,undefined together with the oracle's
 * single C file and run by tests/test_oracle_sanitizers.py.  It calls every
 * oracle entry point on small inputs that reach each branch: all flag
 * patterns of a short window, RoPE at large positions, attention with empty
 * and short prefixes and a row subset, vocabulary statistics with ties and
 * a constant row, commit / select / refill including the fallback, a fully
 * filled window and a missing row.  Any out-of-bounds access, leak or
 * undefined behaviour aborts the run; the few value checks here only guard
 * against a driver that silently does nothing. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int wo_num_threads(void);
double wo_round_storage(double x, int dtype);
int wo_reorder_perm(int W, const uint8_t *filled, int32_t *perm);
void wo_rope(int D, double base, int32_t p, const double *x, double *y);
int wo_reorder(int B, int W, int Hq, int Hkv, int D, int dtype, double base, const uint8_t *filled,
               const int32_t *pos, const double *q, const double *k, const double *v, int32_t *perm,
               double *q_phys, double *k_win, double *v_win);
void wo_attention(int B, int W, int Hq, int Hkv, int D, double scale, const double *q_phys, const double *K,
                  const double *V, const int64_t *kv_off, const int32_t *ctx_len, const int32_t *perm,
                  int64_t n_rows, const int32_t *rows, double *out);
void wo_vocab_stats(int64_t R, int V, const float *logits, int32_t *argmax, double *H);
int wo_select_commit(int B, int W, int V, const float *logits, const int64_t *row_index, int32_t *tok,
                     uint8_t *filled, int32_t *pos, int32_t *ctx_len, int32_t *n_commit, int32_t *committed,
                     int32_t *argmax_out, float *entropy_out, double alpha, double tau, int32_t mask_id,
                     double *margin);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
    CHECK(wo_num_threads() >= 1);
    CHECK(wo_round_storage(1.0 + 1.0 / 512.0, 1) == 1.0);   /* bf16 tie to even */

    /* every flag pattern of a 7-slot window gives a permutation */
    for (int m = 0; m < 128; ++m) {
        uint8_t f[7]; int32_t perm[7]; int seen[7] = {0};
        for (int i = 0; i < 7; ++i) f[i] = (uint8_t)((m >> i) & 1);
        wo_reorder_perm(7, f, perm);
        for (int r = 0; r < 7; ++r) { CHECK(perm[r] >= 0 && perm[r] < 7); seen[perm[r]]++; }
        for (int i = 0; i < 7; ++i) CHECK(seen[i] == 1);
    }
    { double x[8], y[8]; for (int i = 0; i < 8; ++i) x[i] = urand(); wo_rope(8, 1e6, 2147483000, x, y); }

    /* reorder + attention: B=2, W=5, Hq=4, Hkv=2, D=8, prefixes 0 and 9 */
    enum { B = 2, W = 5, HQ = 4, HKV = 2, D = 8 };
    const int32_t ctx[B] = {0, 9};
    uint8_t filled[B * W] = {1, 0, 1, 0, 0, 0, 1, 1, 0, 1};
    int32_t pos[B * W];
    for (int b = 0; b < B; ++b) for (int i = 0; i < W; ++i) pos[b * W + i] = ctx[b] + i;
    double *q = malloc(sizeof(double) * B * W * HQ * D), *k = malloc(sizeof(double) * B * W * HKV * D);
    double *v = malloc(sizeof(double) * B * W * HKV * D), *qp = malloc(sizeof(double) * B * W * HQ * D);
    double *kw = malloc(sizeof(double) * B * W * HKV * D), *vw = malloc(sizeof(double) * B * W * HKV * D);
    for (int i = 0; i < B * W * HQ * D; ++i) q[i] = urand();
    for (int i = 0; i < B * W * HKV * D; ++i) { k[i] = urand(); v[i] = urand(); }
    int32_t perm[B * W];
    CHECK(wo_reorder(B, W, HQ, HKV, D, 1, 1e4, filled, pos, q, k, v, perm, qp, kw, vw) == 0);
    int32_t bad[W] = {3, 4, 4, 5, 6};
    CHECK(wo_reorder(1, W, HQ, HKV, D, 1, 1e4, filled, bad, q, k, v, perm, qp, kw, vw) == -1);
    CHECK(wo_reorder(B, W, HQ, HKV, D, 1, 1e4, filled, pos, q, k, v, perm, qp, kw, vw) == 0);
    /* dense K/V per sequence: prefix rows then the W window rows */
    int64_t off[B]; int64_t total = 0;
    for (int b = 0; b < B; ++b) { off[b] = total; total += ctx[b] + W; }
    double *K = malloc(sizeof(double) * total * HKV * D), *V = malloc(sizeof(double) * total * HKV * D);
    for (int b = 0; b < B; ++b) {
        for (int64_t t = 0; t < ctx[b]; ++t)
            for (int j = 0; j < HKV * D; ++j) {
                K[(off[b] + t) * HKV * D + j] = urand();
                V[(off[b] + t) * HKV * D + j] = urand();
            }
        memcpy(K + (off[b] + ctx[b]) * HKV * D, kw + (size_t)b * W * HKV * D, sizeof(double) * W * HKV * D);
        memcpy(V + (off[b] + ctx[b]) * HKV * D, vw + (size_t)b * W * HKV * D, sizeof(double) * W * HKV * D);
    }
    double *out = malloc(sizeof(double) * B * W * HQ * D);
    wo_attention(B, W, HQ, HKV, D, 0.0, qp, K, V, off, ctx, perm, 0, NULL, out);
    for (int i = 0; i < B * W * HQ * D; ++i) CHECK(isfinite(out[i]));
    const int32_t rows[6] = {0, 0, 0, 1, 4, 3};
    wo_attention(B, W, HQ, HKV, D, 0.25, qp, K, V, off, ctx, perm, 2, rows, out);

    /* vocabulary statistics and commit / select / refill, V = 40 */
    enum { SB = 2, SW = 6, VV = 40 };
    float *lg = malloc(sizeof(float) * SB * SW * VV);
    for (int i = 0; i < SB * SW * VV; ++i) lg[i] = (float)(2.0 * urand());
    for (int i = 0; i < VV; ++i) lg[VV + i] = 0.5f;          /* constant row: H = ln V */
    lg[2 * VV + 3] = lg[2 * VV + 7] = 9.0f;                  /* tied maximum */
    int32_t am[SB * SW]; double H[SB * SW];
    wo_vocab_stats(SB * SW, VV, lg, am, H);
    CHECK(fabs(H[1] - log((double)VV)) < 1e-12 && am[1] == 0 && am[2] == 3);
    int32_t tok[SB * SW], spos[SB * SW], sctx[SB] = {100, 7}, ncom[SB], com[SB * SW], amo[SB * SW];
    uint8_t sf[SB * SW] = {1, 1, 0, 0, 1, 0, 0, 0, 0, 0, 0, 0};
    float ent[SB * SW]; double mg[SB];
    for (int i = 0; i < SB * SW; ++i) { tok[i] = sf[i] ? i : VV; spos[i] = sctx[i / SW] + i % SW; }
    CHECK(wo_select_commit(SB, SW, VV, lg, NULL, tok, sf, spos, sctx, ncom, com, amo, ent, 0.25, 0.5, VV, mg) == 0);
    CHECK(ncom[0] == 2 && ncom[1] == 0);
    /* a fully filled window commits everything; a missing row is an error */
    for (int i = 0; i < SB * SW; ++i) sf[i] = 1;
    CHECK(wo_select_commit(SB, SW, VV, lg, NULL, tok, sf, spos, sctx, ncom, com, NULL, NULL, 0.25, 9.0, VV, NULL) == 0);
    CHECK(ncom[0] == SW && ncom[1] == SW);
    int64_t idx[SB * SW];
    for (int i = 0; i < SB * SW; ++i) { idx[i] = i == 3 ? -1 : i; sf[i] = 0; }
    CHECK(wo_select_commit(SB, SW, VV, lg, idx, tok, sf, spos, sctx, ncom, com, NULL, NULL, 0.25, 9.0, VV, NULL) == -1);

    free(q); free(k); free(v); free(qp); free(kw); free(vw); free(K); free(V); free(out); free(lg);
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
