/*
 * Drives every entry point of the CPU oracle once on small random inputs
 * (ids that are -1, repeated, future or out of range included), for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer.  Exits 0 when every
 * call returns its success code; the sanitizers abort on the first finding.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int nsa_oracle_fwd(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d, int bs, int topk,
                   double scale, const float *q, const float *k, const float *v, const int32_t *block_idx,
                   int64_t nrows, const int64_t *rows, double *out, double *lse);
int64_t nsa_oracle_invert(int64_t T, int B, const int32_t *cu, int Hkv, int bs, int topk,
                          const int32_t *block_idx, int64_t nb_cap, int64_t *offsets, int32_t *entries);
int nsa_oracle_bwd(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d, int bs, int topk,
                   double scale, const float *q, const float *k, const float *v, const int32_t *block_idx,
                   const float *dout, double *dq, double *dk, double *dv);
int nsa_oracle_bwd_dq_rows(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d, int bs, int topk,
                           double scale, const float *q, const float *k, const float *v,
                           const int32_t *block_idx, const float *dout, int64_t nrows, const int64_t *rows,
                           double *dq_rows);
int nsa_oracle_bwd_dkv_blocks(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d, int bs, int topk,
                              double scale, const float *q, const float *k, const float *v,
                              const int32_t *block_idx, const float *dout, int64_t nblocks,
                              const int32_t *blocks_hsj, double *dk_blocks, double *dv_blocks);
int nsa_oracle_window_fwd(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d, int window,
                          double scale, const float *q, const float *k, const float *v, int64_t nrows,
                          const int64_t *rows, double *out, double *lse);
int nsa_oracle_select(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d, int ks, int stride, int bs,
                      int topk, int init_blocks, int local_blocks, double scale, int dtype, const float *q,
                      const float *k, int64_t nrows, const int64_t *rows, int nbmax, int32_t *block_idx,
                      double *imp);

static uint64_t rng_state = 88172645463325252ull;
static uint64_t next_u64(void)  /* xorshift64 (Marsaglia, 2003) */
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}
static float uniform_pm1(void) { return (float)((next_u64() >> 11) * (1.0 / 9007199254740992.0)) * 2.f - 1.f; }

#define CHECK(x)                                                  \
    do {                                                          \
        if ((x) != 0) {                                           \
            fprintf(stderr, "failed: %s (line %d)\n", #x, __LINE__); \
            return 1;                                             \
        }                                                         \
    } while (0)

int main(void)
{
    const int B = 3, Hq = 4, Hkv = 2, d = 64, bs = 32, topk = 6, G = Hq / Hkv;
    const int32_t cu[4] = {0, 100, 100, 257};  /* an empty sequence in the middle */
    const int64_t T = cu[B];
    const int nbmax = 5;                         /* ceil(157 / 32) */
    float *q = malloc(sizeof(float) * T * Hq * d), *k = malloc(sizeof(float) * T * Hkv * d);
    float *v = malloc(sizeof(float) * T * Hkv * d), *dout = malloc(sizeof(float) * T * Hq * d);
    int32_t *bi = malloc(sizeof(int32_t) * T * Hkv * topk);
    for (int64_t i = 0; i < T * Hq * d; ++i) { q[i] = uniform_pm1(); dout[i] = uniform_pm1(); }
    for (int64_t i = 0; i < T * Hkv * d; ++i) { k[i] = uniform_pm1(); v[i] = uniform_pm1(); }
    for (int64_t i = 0; i < T * Hkv * topk; ++i) bi[i] = (int32_t)(next_u64() % (nbmax + 2)) - 1;

    double *out = malloc(sizeof(double) * T * Hq * d), *lse = malloc(sizeof(double) * T * Hq);
    CHECK(nsa_oracle_fwd(T, B, cu, Hq, Hkv, d, bs, topk, 0.125, q, k, v, bi, 0, NULL, out, lse));
    const int64_t rows[4] = {0, 7, 2 * 100 + 1, 2 * 256 + 1};
    double *out_r = malloc(sizeof(double) * 4 * G * d), *lse_r = malloc(sizeof(double) * 4 * G);
    CHECK(nsa_oracle_fwd(T, B, cu, Hq, Hkv, d, bs, topk, 0.125, q, k, v, bi, 4, rows, out_r, lse_r));

    const int64_t cap = T / bs + B;
    int64_t *offsets = malloc(sizeof(int64_t) * (Hkv * cap + 1));
    int32_t *entries = malloc(sizeof(int32_t) * T * Hkv * topk);
    if (nsa_oracle_invert(T, B, cu, Hkv, bs, topk, bi, cap, offsets, entries) < 0) return 1;

    double *dq = malloc(sizeof(double) * T * Hq * d), *dk = malloc(sizeof(double) * T * Hkv * d);
    double *dv = malloc(sizeof(double) * T * Hkv * d);
    CHECK(nsa_oracle_bwd(T, B, cu, Hq, Hkv, d, bs, topk, 0.125, q, k, v, bi, dout, dq, dk, dv));
    double *dq_r = malloc(sizeof(double) * 4 * G * d);
    CHECK(nsa_oracle_bwd_dq_rows(T, B, cu, Hq, Hkv, d, bs, topk, 0.125, q, k, v, bi, dout, 4, rows, dq_r));
    const int32_t blocks[9] = {0, 0, 0, 1, 2, 4, 1, 0, 3};  /* (h, s, j); block 4 of s 2 is partial */
    double *dkb = malloc(sizeof(double) * 3 * bs * d), *dvb = malloc(sizeof(double) * 3 * bs * d);
    CHECK(nsa_oracle_bwd_dkv_blocks(T, B, cu, Hq, Hkv, d, bs, topk, 0.125, q, k, v, bi, dout, 3, blocks, dkb,
                                    dvb));
    CHECK(nsa_oracle_window_fwd(T, B, cu, Hq, Hkv, d, 40, 0.125, q, k, v, 0, NULL, out, lse));
    CHECK(nsa_oracle_window_fwd(T, B, cu, Hq, Hkv, d, 40, 0.125, q, k, v, 4, rows, out_r, lse_r));

    /* index producer: kernel 32, stride 16, blocks of 64 */
    const int sel_nbmax = 3;
    int32_t *sel = malloc(sizeof(int32_t) * T * Hkv * topk);
    double *imp = malloc(sizeof(double) * T * Hkv * sel_nbmax);
    CHECK(nsa_oracle_select(T, B, cu, Hq, Hkv, d, 32, 16, 64, topk, 1, 2, 0.125, 1, q, k, 0, NULL, sel_nbmax,
                            sel, imp));
    CHECK(nsa_oracle_select(T, B, cu, Hq, Hkv, d, 32, 16, 64, topk, 1, 2, 0.125, 2, q, k, 4, rows, sel_nbmax,
                            sel, imp));

    double acc = 0.0;
    for (int64_t i = 0; i < T * Hq; ++i) acc += isfinite(lse[i]) ? lse[i] : 0.0;
    printf("oracle driver ok (checksum %.6f)\n", acc);
    free(q); free(k); free(v); free(dout); free(bi); free(out); free(lse); free(out_r); free(lse_r);
    free(offsets); free(entries); free(dq); free(dk); free(dv); free(dq_r); free(dkb); free(dvb);
    free(sel); free(imp);
    return 0;
}
