/*
 * nsa_oracle.c -- reference oracle for NSA selected-block attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow CPU implementation in
 * double precision, written from the definition of the operation.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg load it;
 * the product (HIP) path never calls it and shares no code, header or table
 * with it.
 *
 * What is computed.  Native Sparse Attention's selection branch: each query
 * token attends, for every query head of its GQA group, only to the keys of
 * the `topk` blocks of `block_size` tokens that its block list names
 * (Flash-Sparse-Attention project page, agentlenshq
 * "Relaxed-System-Lab/Flash-Sparse-Attention": "Quick start" constructor
 * arguments block_size / topk / init_blocks / local_blocks, and the varlen
 * packing by cu_seqlens; q2bstudio "FSA: efficient implementation of native
 * sparse attention", first paragraph, for the GQA grouping).  FSA's loop
 * reordering and its reduction / online-softmax kernels ("Key features",
 * optimised-kernels row) compute exactly this result up to rounding, so the
 * oracle is the plain definition, with no blocking, no online softmax and no
 * partial results.  The pages leave the following open; the readings taken:
 *
 *   - selected set S(t,h): the distinct ids j in block_idx[t][h][:] with
 *     0 <= j <= b(t); -1, future blocks and repeats name no extra keys;
 *     the slot of a block is its first position in the row;
 *   - keys: every position p of a selected block with p < L_s and p <= i
 *     (causal, diagonal included), never crossing a sequence;
 *   - GQA: query head qh uses kv head qh / G (contiguous groups);
 *   - lse = m + ln(sum exp(s - m)) in natural log; an empty key set gives
 *     out = 0 and lse = -inf.
 *
 * Layouts (row-major): q [T][Hq][d], k and v [T][Hkv][d], block_idx
 * [T][Hkv][topk] int32, cu_seqlens [B+1] int32, out [rows][G][d] and
 * lse [rows][G] in double, one row per (t, h) pair.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Sequence holding token t: the s with cu[s] <= t < cu[s+1]. */
static int seq_of(const int32_t *cu, int B, int64_t t)
{
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Distinct valid blocks of one row (0 <= j <= b_max), first slot of each,
 * sorted by block id.  Returns how many. */
static int selected_blocks(const int32_t *row, int topk, int b_max,
                           int *blocks, int *slots)
{
    int n = 0;
    for (int k = 0; k < topk; ++k) {
        int j = row[k];
        if (j < 0 || j > b_max) continue;
        int seen = 0;
        for (int m = 0; m < n; ++m)
            if (blocks[m] == j) { seen = 1; break; }
        if (seen) continue;
        blocks[n] = j;
        slots[n] = k;
        ++n;
    }
    for (int a = 1; a < n; ++a) {          /* insertion sort by block id */
        int bj = blocks[a], sj = slots[a], c = a - 1;
        while (c >= 0 && blocks[c] > bj) {
            blocks[c + 1] = blocks[c];
            slots[c + 1] = slots[c];
            --c;
        }
        blocks[c + 1] = bj;
        slots[c + 1] = sj;
    }
    return n;
}

/* Key positions (global token ids, ascending) visible to token t of sequence
 * s under row (t, h).  Returns how many. */
static int key_set(const int32_t *cu, int B, int bs, int topk,
                   const int32_t *block_idx, int Hkv, int64_t t, int h,
                   int64_t *keys, int *blocks, int *slots)
{
    int s = seq_of(cu, B, t);
    int64_t c = cu[s], L = (int64_t)cu[s + 1] - c, i = t - c;
    int b = (int)(i / bs);
    const int32_t *row = block_idx + ((size_t)t * Hkv + h) * topk;
    int nsel = selected_blocks(row, topk, b, blocks, slots);
    int n = 0;
    for (int a = 0; a < nsel; ++a) {
        int64_t p0 = (int64_t)blocks[a] * bs, p1 = p0 + bs;
        if (p1 > L) p1 = L;
        for (int64_t p = p0; p < p1 && p <= i; ++p)
            keys[n++] = c + p;
    }
    return n;
}

/*
 * Forward.  rows == NULL computes every (t, h) row and writes out/lse in the
 * natural order (out [T][Hq][d], lse [T][Hq]); otherwise rows[r] = t*Hkv + h
 * names the rows to compute and out/lse are [nrows][G][d] / [nrows][G].
 * Inputs are float (exact values of the generated data), arithmetic is
 * double.  Returns 0, or -1 on bad arguments.
 */
int nsa_oracle_fwd(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                   int bs, int topk, double scale,
                   const float *q, const float *k, const float *v,
                   const int32_t *block_idx,
                   int64_t nrows, const int64_t *rows,
                   double *out, double *lse)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || bs < 1 || topk < 1)
        return -1;
    const int G = Hq / Hkv;
    const int64_t n_rows = rows ? nrows : T * Hkv;
    const int max_keys = topk * bs;
    int bad = 0;

#pragma omp parallel
    {
        int64_t *keys = malloc(sizeof(int64_t) * (size_t)max_keys);
        double *sc = malloc(sizeof(double) * (size_t)max_keys);
        int *blocks = malloc(sizeof(int) * (size_t)topk);
        int *slots = malloc(sizeof(int) * (size_t)topk);
        if (!keys || !sc || !blocks || !slots) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 64)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t th = rows ? rows[r] : r;
                int64_t t = th / Hkv;
                int h = (int)(th % Hkv);
                int n = key_set(cu, B, bs, topk, block_idx, Hkv, t, h, keys, blocks, slots);
                for (int g = 0; g < G; ++g) {
                    int qh = h * G + g;
                    const float *qr = q + ((size_t)t * Hq + qh) * d;
                    double *o = out + ((size_t)r * G + g) * d;
                    double *ls = lse + (size_t)r * G + g;
                    for (int e = 0; e < d; ++e) o[e] = 0.0;
                    if (n == 0) { *ls = -INFINITY; continue; }
                    double m = -INFINITY;
                    for (int a = 0; a < n; ++a) {
                        const float *kr = k + ((size_t)keys[a] * Hkv + h) * d;
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e) acc += (double)qr[e] * (double)kr[e];
                        sc[a] = scale * acc;
                        if (sc[a] > m) m = sc[a];
                    }
                    double l = 0.0;
                    for (int a = 0; a < n; ++a) {
                        double w = exp(sc[a] - m);
                        const float *vr = v + ((size_t)keys[a] * Hkv + h) * d;
                        l += w;
                        for (int e = 0; e < d; ++e) o[e] += w * (double)vr[e];
                    }
                    for (int e = 0; e < d; ++e) o[e] /= l;
                    *ls = m + log(l);
                }
            }
        }
        free(keys); free(sc); free(blocks); free(slots);
    }
    return bad ? -1 : 0;
}

/*
 * Index inversion: per-row block lists -> per-block token lists (CSR).
 * Bucket of (t, h, j) is h*nb_cap + blkoff[s] + j, where blkoff[s] is the
 * number of blocks of the sequences before s (nb_s = ceil(L_s / bs)) and
 * nb_cap = T / bs + B bounds the total block count.  Each bucket lists
 * t*topk + slot for the t that select it, ascending in t.  offsets has
 * Hkv*nb_cap + 1 entries (empty buckets repeat their start; the last entry
 * is nnz).  entries must hold T*Hkv*topk values.  Returns nnz, or -1.
 */
int64_t nsa_oracle_invert(int64_t T, int B, const int32_t *cu, int Hkv, int bs,
                          int topk, const int32_t *block_idx, int64_t nb_cap,
                          int64_t *offsets, int32_t *entries)
{
    if (T < 0 || B < 1 || Hkv < 1 || bs < 1 || topk < 1) return -1;
    int64_t *blkoff = malloc(sizeof(int64_t) * (size_t)(B + 1));
    int *blocks = malloc(sizeof(int) * (size_t)topk);
    int *slots = malloc(sizeof(int) * (size_t)topk);
    int64_t nbk = (int64_t)Hkv * nb_cap;
    int64_t *cursor = calloc((size_t)nbk + 1, sizeof(int64_t));
    if (!blkoff || !blocks || !slots || !cursor) {
        free(blkoff); free(blocks); free(slots); free(cursor);
        return -1;
    }
    blkoff[0] = 0;
    for (int s = 0; s < B; ++s)
        blkoff[s + 1] = blkoff[s] + ((int64_t)cu[s + 1] - cu[s] + bs - 1) / bs;
    if (blkoff[B] > nb_cap) {
        free(blkoff); free(blocks); free(slots); free(cursor);
        return -1;
    }

    /* counts */
    for (int64_t b = 0; b <= nbk; ++b) offsets[b] = 0;
    for (int h = 0; h < Hkv; ++h)
        for (int64_t t = 0; t < T; ++t) {
            int s = seq_of(cu, B, t);
            int bt = (int)((t - cu[s]) / bs);
            const int32_t *row = block_idx + ((size_t)t * Hkv + h) * topk;
            int n = selected_blocks(row, topk, bt, blocks, slots);
            for (int a = 0; a < n; ++a)
                offsets[h * nb_cap + blkoff[s] + blocks[a] + 1] += 1;
        }
    for (int64_t b = 0; b < nbk; ++b) offsets[b + 1] += offsets[b];
    for (int64_t b = 0; b < nbk; ++b) cursor[b] = offsets[b];

    /* fill, t ascending within every bucket */
    for (int h = 0; h < Hkv; ++h)
        for (int64_t t = 0; t < T; ++t) {
            int s = seq_of(cu, B, t);
            int bt = (int)((t - cu[s]) / bs);
            const int32_t *row = block_idx + ((size_t)t * Hkv + h) * topk;
            int n = selected_blocks(row, topk, bt, blocks, slots);
            for (int a = 0; a < n; ++a) {
                int64_t bkt = h * nb_cap + blkoff[s] + blocks[a];
                entries[cursor[bkt]++] = (int32_t)(t * topk + slots[a]);
            }
        }
    int64_t nnz = offsets[nbk];
    free(blkoff); free(blocks); free(slots); free(cursor);
    return nnz;
}

/*
 * Backward of the forward above for upstream gradient dO [T][Hq][d]
 * (Flash-Sparse-Attention project page, "Key features", training row: the
 * full backward pass is supported).  With P_p = exp(s_p - lse), out the
 * oracle's own forward output and D = sum_e dO[e] * out[e]:
 *   dV[p] += P_p dO,  dS_p = P_p (dO . v[p] - D),
 *   dQ = scale * sum_p dS_p k[p],  dK[p] += scale * dS_p q.
 * Every (t, qh) row is processed in ascending t, then ascending qh; one
 * thread owns each kv head, so the accumulation order is that loop order.
 * dq [T][Hq][d], dk and dv [T][Hkv][d] are written in full.
 */
int nsa_oracle_bwd(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                   int bs, int topk, double scale,
                   const float *q, const float *k, const float *v,
                   const int32_t *block_idx, const float *dout,
                   double *dq, double *dk, double *dv)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || bs < 1 || topk < 1)
        return -1;
    const int G = Hq / Hkv;
    const int max_keys = topk * bs;
    int bad = 0;
    memset(dq, 0, sizeof(double) * (size_t)T * Hq * d);
    memset(dk, 0, sizeof(double) * (size_t)T * Hkv * d);
    memset(dv, 0, sizeof(double) * (size_t)T * Hkv * d);

#pragma omp parallel for schedule(static, 1)
    for (int h = 0; h < Hkv; ++h) {
        int64_t *keys = malloc(sizeof(int64_t) * (size_t)max_keys);
        double *sc = malloc(sizeof(double) * (size_t)max_keys);
        double *o = malloc(sizeof(double) * (size_t)d);
        int *blocks = malloc(sizeof(int) * (size_t)topk);
        int *slots = malloc(sizeof(int) * (size_t)topk);
        if (!keys || !sc || !o || !blocks || !slots) {
#pragma omp atomic write
            bad = 1;
        } else {
            for (int64_t t = 0; t < T; ++t) {
                int n = key_set(cu, B, bs, topk, block_idx, Hkv, t, h, keys, blocks, slots);
                if (n == 0) continue;
                for (int g = 0; g < G; ++g) {
                    int qh = h * G + g;
                    const float *qr = q + ((size_t)t * Hq + qh) * d;
                    const float *dor = dout + ((size_t)t * Hq + qh) * d;
                    double m = -INFINITY;
                    for (int a = 0; a < n; ++a) {
                        const float *kr = k + ((size_t)keys[a] * Hkv + h) * d;
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e) acc += (double)qr[e] * (double)kr[e];
                        sc[a] = scale * acc;
                        if (sc[a] > m) m = sc[a];
                    }
                    double l = 0.0;
                    for (int e = 0; e < d; ++e) o[e] = 0.0;
                    for (int a = 0; a < n; ++a) {
                        double w = exp(sc[a] - m);
                        const float *vr = v + ((size_t)keys[a] * Hkv + h) * d;
                        l += w;
                        for (int e = 0; e < d; ++e) o[e] += w * (double)vr[e];
                    }
                    for (int e = 0; e < d; ++e) o[e] /= l;
                    double lse = m + log(l);
                    double D = 0.0;
                    for (int e = 0; e < d; ++e) D += (double)dor[e] * o[e];
                    double *dqr = dq + ((size_t)t * Hq + qh) * d;
                    for (int a = 0; a < n; ++a) {
                        double P = exp(sc[a] - lse);
                        const float *kr = k + ((size_t)keys[a] * Hkv + h) * d;
                        const float *vr = v + ((size_t)keys[a] * Hkv + h) * d;
                        double *dkr = dk + ((size_t)keys[a] * Hkv + h) * d;
                        double *dvr = dv + ((size_t)keys[a] * Hkv + h) * d;
                        double dP = 0.0;
                        for (int e = 0; e < d; ++e) dP += (double)dor[e] * (double)vr[e];
                        double dS = P * (dP - D);
                        for (int e = 0; e < d; ++e) {
                            dvr[e] += P * (double)dor[e];
                            dqr[e] += scale * dS * (double)kr[e];
                            dkr[e] += scale * dS * (double)qr[e];
                        }
                    }
                }
            }
        }
        free(keys); free(sc); free(o); free(blocks); free(slots);
    }
    return bad ? -1 : 0;
}

/*
 * Sliding-window branch ([FSA-README] "Quick start": window_size, the third
 * NSA branch beside compression and selection).  Reading taken: token i of a
 * sequence attends, for each query head, to the keys p of its own sequence
 * with i - window < p <= i (itself included), with the same scale, GQA
 * mapping and natural-log lse as the selection branch.  rows / out / lse as
 * in nsa_oracle_fwd.
 */
int nsa_oracle_window_fwd(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                          int window, double scale,
                          const float *q, const float *k, const float *v,
                          int64_t nrows, const int64_t *rows,
                          double *out, double *lse)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || window < 1)
        return -1;
    const int G = Hq / Hkv;
    const int64_t n_rows = rows ? nrows : T * Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *sc = malloc(sizeof(double) * (size_t)window);
        if (!sc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 64)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t th = rows ? rows[r] : r;
                int64_t t = th / Hkv;
                int h = (int)(th % Hkv);
                int s = seq_of(cu, B, t);
                int64_t c = cu[s], i = t - c;
                int64_t p0 = i - window + 1 < 0 ? 0 : i - window + 1;
                int n = (int)(i - p0 + 1);
                for (int g = 0; g < G; ++g) {
                    int qh = h * G + g;
                    const float *qr = q + ((size_t)t * Hq + qh) * d;
                    double *o = out + ((size_t)r * G + g) * d;
                    double m = -INFINITY;
                    for (int a = 0; a < n; ++a) {
                        const float *kr = k + ((size_t)(c + p0 + a) * Hkv + h) * d;
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e) acc += (double)qr[e] * (double)kr[e];
                        sc[a] = scale * acc;
                        if (sc[a] > m) m = sc[a];
                    }
                    double l = 0.0;
                    for (int e = 0; e < d; ++e) o[e] = 0.0;
                    for (int a = 0; a < n; ++a) {
                        double w = exp(sc[a] - m);
                        const float *vr = v + ((size_t)(c + p0 + a) * Hkv + h) * d;
                        l += w;
                        for (int e = 0; e < d; ++e) o[e] += w * (double)vr[e];
                    }
                    for (int e = 0; e < d; ++e) o[e] /= l;
                    lse[(size_t)r * G + g] = m + log(l);
                }
            }
        }
        free(sc);
    }
    return bad ? -1 : 0;
}

/*
 * The backward above, restricted so that full-size workloads can be checked
 * on samples.  Same definitions and the same (t ascending, qh ascending)
 * accumulation order; lse and out of every row involved are the oracle's own.
 *
 * nsa_oracle_bwd_dq_rows: dq for the listed rows (rows[r] = t*Hkv + h), all G
 * query heads of each: dq_rows [nrows][G][d].
 *
 * nsa_oracle_bwd_dkv_blocks: dk and dv of the keys of the listed blocks
 * (blocks[3*i] = h, blocks[3*i+1] = s, blocks[3*i+2] = j): for each block,
 * every row (t, h) of sequence s that selects j contributes.  The rows are
 * cut into NCHUNK contiguous runs of t, each summed in ascending t, and the
 * run sums are added in run order (a block that every token selects has
 * tens of thousands of rows, each needing its full forward).
 * Output dk_blocks, dv_blocks [nblocks][bs][d]; keys past the end of the
 * sequence are 0.
 */
static void row_forward(int64_t t, int h, int qh, int n, const int64_t *keys, int Hq, int Hkv,
                        int d, double scale, const float *q, const float *k, const float *v,
                        const float *dout, double *sc, double *o, double *lse_out, double *D_out)
{
    const float *qr = q + ((size_t)t * Hq + qh) * d;
    double m = -INFINITY;
    for (int a = 0; a < n; ++a) {
        const float *kr = k + ((size_t)keys[a] * Hkv + h) * d;
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += (double)qr[e] * (double)kr[e];
        sc[a] = scale * acc;
        if (sc[a] > m) m = sc[a];
    }
    double l = 0.0;
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int a = 0; a < n; ++a) {
        double w = exp(sc[a] - m);
        const float *vr = v + ((size_t)keys[a] * Hkv + h) * d;
        l += w;
        for (int e = 0; e < d; ++e) o[e] += w * (double)vr[e];
    }
    for (int e = 0; e < d; ++e) o[e] /= l;
    *lse_out = m + log(l);
    const float *dor = dout + ((size_t)t * Hq + qh) * d;
    double D = 0.0;
    for (int e = 0; e < d; ++e) D += (double)dor[e] * o[e];
    *D_out = D;
}

int nsa_oracle_bwd_dq_rows(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                           int bs, int topk, double scale,
                           const float *q, const float *k, const float *v,
                           const int32_t *block_idx, const float *dout,
                           int64_t nrows, const int64_t *rows, double *dq_rows)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || bs < 1 || topk < 1) return -1;
    const int G = Hq / Hkv;
    const int max_keys = topk * bs;
    int bad = 0;
#pragma omp parallel
    {
        int64_t *keys = malloc(sizeof(int64_t) * (size_t)max_keys);
        double *sc = malloc(sizeof(double) * (size_t)max_keys);
        double *o = malloc(sizeof(double) * (size_t)d);
        int *blocks = malloc(sizeof(int) * (size_t)topk);
        int *slots = malloc(sizeof(int) * (size_t)topk);
        if (!keys || !sc || !o || !blocks || !slots) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t t = rows[r] / Hkv;
                int h = (int)(rows[r] % Hkv);
                int n = key_set(cu, B, bs, topk, block_idx, Hkv, t, h, keys, blocks, slots);
                for (int g = 0; g < G; ++g) {
                    int qh = h * G + g;
                    double *dqr = dq_rows + ((size_t)r * G + g) * d;
                    for (int e = 0; e < d; ++e) dqr[e] = 0.0;
                    if (n == 0) continue;
                    double lse, D;
                    row_forward(t, h, qh, n, keys, Hq, Hkv, d, scale, q, k, v, dout, sc, o, &lse, &D);
                    const float *dor = dout + ((size_t)t * Hq + qh) * d;
                    for (int a = 0; a < n; ++a) {
                        double P = exp(sc[a] - lse);
                        const float *kr = k + ((size_t)keys[a] * Hkv + h) * d;
                        const float *vr = v + ((size_t)keys[a] * Hkv + h) * d;
                        double dP = 0.0;
                        for (int e = 0; e < d; ++e) dP += (double)dor[e] * (double)vr[e];
                        double dS = P * (dP - D);
                        for (int e = 0; e < d; ++e) dqr[e] += scale * dS * (double)kr[e];
                    }
                }
            }
        }
        free(keys); free(sc); free(o); free(blocks); free(slots);
    }
    return bad ? -1 : 0;
}

#define NCHUNK 64

int nsa_oracle_bwd_dkv_blocks(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                              int bs, int topk, double scale,
                              const float *q, const float *k, const float *v,
                              const int32_t *block_idx, const float *dout,
                              int64_t nblocks, const int32_t *blocks_hsj,
                              double *dk_blocks, double *dv_blocks)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || bs < 1 || topk < 1) return -1;
    const int G = Hq / Hkv;
    const int max_keys = topk * bs;
    const size_t bd = (size_t)bs * d;
    double *run_k = calloc((size_t)NCHUNK * bd, sizeof(double));
    double *run_v = calloc((size_t)NCHUNK * bd, sizeof(double));
    if (!run_k || !run_v) {
        free(run_k); free(run_v);
        return -1;
    }
    int bad = 0;
    for (int64_t ib = 0; ib < nblocks; ++ib) {
        int h = blocks_hsj[3 * ib], s = blocks_hsj[3 * ib + 1], j = blocks_hsj[3 * ib + 2];
        int64_t c = cu[s], L = (int64_t)cu[s + 1] - c;
        int64_t p0 = c + (int64_t)j * bs;
#pragma omp parallel
        {
            int64_t *keys = malloc(sizeof(int64_t) * (size_t)max_keys);
            double *sc = malloc(sizeof(double) * (size_t)max_keys);
            double *o = malloc(sizeof(double) * (size_t)d);
            int *blocks = malloc(sizeof(int) * (size_t)topk);
            int *slots = malloc(sizeof(int) * (size_t)topk);
            if (!keys || !sc || !o || !blocks || !slots) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int r = 0; r < NCHUNK; ++r) {
                    double *dkb = run_k + (size_t)r * bd;
                    double *dvb = run_v + (size_t)r * bd;
                    for (size_t x = 0; x < bd; ++x) dkb[x] = dvb[x] = 0.0;
                    int64_t t0 = c + L * r / NCHUNK, t1 = c + L * (r + 1) / NCHUNK;
                    for (int64_t t = t0; t < t1; ++t) {
                        int n = key_set(cu, B, bs, topk, block_idx, Hkv, t, h, keys, blocks, slots);
                        int sel = 0;
                        for (int a = 0; a < n; ++a)
                            if (keys[a] >= p0 && keys[a] < p0 + bs) { sel = 1; break; }
                        if (!sel) continue;
                        for (int g = 0; g < G; ++g) {
                            int qh = h * G + g;
                            double lse, D;
                            row_forward(t, h, qh, n, keys, Hq, Hkv, d, scale, q, k, v, dout, sc, o, &lse, &D);
                            const float *qr = q + ((size_t)t * Hq + qh) * d;
                            const float *dor = dout + ((size_t)t * Hq + qh) * d;
                            for (int a = 0; a < n; ++a) {
                                if (keys[a] < p0 || keys[a] >= p0 + bs) continue;
                                double P = exp(sc[a] - lse);
                                const float *vr = v + ((size_t)keys[a] * Hkv + h) * d;
                                double dP = 0.0;
                                for (int e = 0; e < d; ++e) dP += (double)dor[e] * (double)vr[e];
                                double dS = P * (dP - D);
                                double *dkr = dkb + (size_t)(keys[a] - p0) * d;
                                double *dvr = dvb + (size_t)(keys[a] - p0) * d;
                                for (int e = 0; e < d; ++e) {
                                    dvr[e] += P * (double)dor[e];
                                    dkr[e] += scale * dS * (double)qr[e];
                                }
                            }
                        }
                    }
                }
            }
            free(keys); free(sc); free(o); free(blocks); free(slots);
        }
        double *dkb = dk_blocks + (size_t)ib * bd;
        double *dvb = dv_blocks + (size_t)ib * bd;
        for (size_t x = 0; x < bd; ++x) dkb[x] = dvb[x] = 0.0;
        for (int r = 0; r < NCHUNK; ++r)
            for (size_t x = 0; x < bd; ++x) {
                dkb[x] += run_k[(size_t)r * bd + x];
                dvb[x] += run_v[(size_t)r * bd + x];
            }
    }
    free(run_k); free(run_v);
    return bad ? -1 : 0;
}

/*
 * dk and dv of every key, from each row's log-sum-exp and D = dout . out
 * (lse and D given as [T][Hq], as the forward computes them).  With
 * P_p = exp(s_p - lse) and dS_p = P_p (dout . v_p - D), dk_p collects
 * scale dS_p q and dv_p collects P_p dout over every row (t, qh) whose key set
 * holds p: the rows of p's kv head whose kept blocks include p's block j, at
 * p <= i.  One thread per (kv head, sequence, key block); its rows in
 * ascending t, then qh, so every sum has that fixed order.  Keys outside
 * every sequence keep dk = dv = 0.
 */
int nsa_oracle_bwd_dkv_all(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                           int bs, int topk, double scale,
                           const float *q, const float *k, const float *v,
                           const int32_t *block_idx, const float *dout,
                           const double *lse, const double *Drow,
                           double *dk, double *dv)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || bs < 1 || topk < 1) return -1;
    const int G = Hq / Hkv;
    memset(dk, 0, sizeof(double) * (size_t)T * Hkv * d);
    memset(dv, 0, sizeof(double) * (size_t)T * Hkv * d);
    int64_t *first = malloc(sizeof(int64_t) * (size_t)(B + 1));  /* first global block of each sequence */
    if (!first) return -1;
    first[0] = 0;
    for (int s = 0; s < B; ++s) {
        int64_t L = (int64_t)cu[s + 1] - cu[s];
        first[s + 1] = first[s] + (L > 0 ? (L + bs - 1) / bs : 0);
    }
    const int64_t ntask = first[B] * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < ntask; ++task) {
        const int h = (int)(task % Hkv);
        const int64_t gb = task / Hkv;
        int s = 0;
        while (first[s + 1] <= gb) ++s;
        const int j = (int)(gb - first[s]);
        const int64_t c = cu[s], end = cu[s + 1];
        const int64_t p0 = c + (int64_t)j * bs, p1 = p0 + bs < end ? p0 + bs : end;
        for (int64_t t = p0; t < end; ++t) {  /* every later token has j <= its own block */
            const int32_t *row = block_idx + ((size_t)t * Hkv + h) * topk;
            int sel = 0;
            for (int a = 0; a < topk; ++a)
                if (row[a] == j) { sel = 1; break; }
            if (!sel) continue;
            const int64_t pend = t + 1 < p1 ? t + 1 : p1;  /* keys p <= i */
            for (int g = 0; g < G; ++g) {
                const int qh = h * G + g;
                const float *qr = q + ((size_t)t * Hq + qh) * d;
                const float *dor = dout + ((size_t)t * Hq + qh) * d;
                const double l = lse[(size_t)t * Hq + qh], D = Drow[(size_t)t * Hq + qh];
                for (int64_t p = p0; p < pend; ++p) {
                    const float *kr = k + ((size_t)p * Hkv + h) * d;
                    const float *vr = v + ((size_t)p * Hkv + h) * d;
                    double sc = 0.0, dP = 0.0;
                    for (int e = 0; e < d; ++e) {
                        sc += (double)qr[e] * (double)kr[e];
                        dP += (double)dor[e] * (double)vr[e];
                    }
                    const double P = exp(scale * sc - l);
                    const double dS = P * (dP - D);
                    double *dkr = dk + ((size_t)p * Hkv + h) * d;
                    double *dvr = dv + ((size_t)p * Hkv + h) * d;
                    for (int e = 0; e < d; ++e) {
                        dvr[e] += P * (double)dor[e];
                        dkr[e] += scale * dS * (double)qr[e];
                    }
                }
            }
        }
    }
    free(first);
    return 0;
}

/*
 * Index producer: the selection branch's block list (block_idx) from
 * compressed attention.  The pages name the module's arguments -- kernel
 * size 32 and stride 16 for the compressed keys, block_size, topk,
 * init_blocks 1 and local_blocks 2 (Flash-Sparse-Attention project page,
 * "Quick start", step 2) -- but print no formula, so the plainest reading of
 * each step is taken:
 *
 *   - compressed keys: window c of a sequence covers positions
 *     [c*stride, c*stride + ks); there are (L - ks) / stride + 1 windows
 *     (none when L < ks).  Its key is the mean of the window's k rows (no
 *     learned weights), accumulated in fp32 in position order, divided by ks
 *     in fp32 and rounded to nearest-even in the input format (dtype 1 bf16,
 *     2 fp16, 0 kept in fp32): the compressed keys are activations;
 *   - compressed attention: query (t, qh) at local position i sees window c
 *     iff c*stride + ks - 1 <= i; p = softmax over the visible windows of
 *     scale * q . kc (none visible: p = 0);
 *   - block importance: imp[j] = sum over the G query heads of the kv group
 *     and over the visible windows that overlap block j (positions
 *     [j*bs, (j+1)*bs)) of p.  A window across a block boundary counts for
 *     both blocks.  One list per (token, kv head), as block_idx's layout has;
 *   - list: first the init blocks 0 .. init-1, then the local blocks b,
 *     b-1, .., b-local+1 (b = i / bs; ids outside [0, b] and repeats
 *     skipped), then the other blocks of [0, b] by importance, largest first
 *     (ties: lower id first), up to topk ids; -1 fills the rest.
 *
 * Scores, softmax and importance are in double precision.  Rows as in
 * nsa_oracle_fwd (rows[r] = t*Hkv + h, or every row when rows is NULL).
 * Output: block_idx [nrows][topk]; imp (optional) [nrows][nbmax], -1 for
 * blocks past b.  Returns -1 on bad arguments.
 */
static double round_to_format(float x, int dtype)
{
    if (dtype == 0 || x == 0.0f || !isfinite(x)) return (double)x;
    int e;
    double m = frexp((double)x, &e);          /* x = m * 2^e, 0.5 <= |m| < 1 */
    int bits = dtype == 1 ? 8 : 11;           /* significant bits of bf16 / fp16 */
    int q = e - bits;                         /* exponent of the last kept bit */
    if (dtype == 2 && q < -24) q = -24;       /* fp16 subnormal quantum */
    double scaled = ldexp((double)x, -q);
    double r = nearbyint(scaled);             /* round half to even (default mode) */
    return ldexp(r, q);
}

int nsa_oracle_select(int64_t T, int B, const int32_t *cu, int Hq, int Hkv, int d,
                      int ks, int stride, int bs, int topk, int init_blocks, int local_blocks,
                      double scale, int dtype, const float *q, const float *k,
                      int64_t nrows, const int64_t *rows, int nbmax,
                      int32_t *block_idx, double *imp)
{
    if (T < 0 || B < 1 || Hkv < 1 || Hq % Hkv || d < 1 || ks < 1 || stride < 1 || bs < 1 ||
        topk < 1 || init_blocks < 0 || local_blocks < 0 || nbmax < 1)
        return -1;
    const int G = Hq / Hkv;
    /* compressed keys of every sequence, window and kv head */
    int64_t *cbase = malloc(sizeof(int64_t) * (size_t)(B + 1));
    if (!cbase) return -1;
    cbase[0] = 0;
    for (int s = 0; s < B; ++s) {
        int64_t L = cu[s + 1] - cu[s];
        cbase[s + 1] = cbase[s] + (L >= ks ? (L - ks) / stride + 1 : 0);
    }
    double *kc = malloc(sizeof(double) * (size_t)(cbase[B] * Hkv * d + 1));
    if (!kc) { free(cbase); return -1; }
    for (int s = 0; s < B; ++s)
        for (int64_t c = 0; c < cbase[s + 1] - cbase[s]; ++c)
            for (int h = 0; h < Hkv; ++h)
                for (int e = 0; e < d; ++e) {
                    float acc = 0.0f;
                    for (int a = 0; a < ks; ++a)
                        acc += k[((size_t)(cu[s] + c * stride + a) * Hkv + h) * d + e];
                    kc[((size_t)(cbase[s] + c) * Hkv + h) * d + e] = round_to_format(acc / (float)ks, dtype);
                }
    const int64_t n_rows = rows ? nrows : T * Hkv;
    int bad = 0;
#pragma omp parallel
    {
        int64_t ncmax = 0;
        for (int s = 0; s < B; ++s)
            if (cbase[s + 1] - cbase[s] > ncmax) ncmax = cbase[s + 1] - cbase[s];
        double *p = malloc(sizeof(double) * (size_t)(ncmax + 1));
        double *im = malloc(sizeof(double) * (size_t)nbmax);
        char *taken = malloc((size_t)nbmax);
        if (!p || !im || !taken) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t th = rows ? rows[r] : r;
                int64_t t = th / Hkv;
                int h = (int)(th % Hkv);
                int s = seq_of(cu, B, t);
                int64_t i = t - cu[s];
                int b = (int)(i / bs);
                int32_t *out = block_idx + (size_t)r * topk;
                for (int x = 0; x < topk; ++x) out[x] = -1;
                if (b >= nbmax || t >= cu[B]) continue;
                for (int j = 0; j < nbmax; ++j) im[j] = j <= b ? 0.0 : -1.0;
                /* visible windows: c*stride + ks - 1 <= i */
                int64_t nvis = i - ks + 1 < 0 ? 0 : (i - ks + 1) / stride + 1;
                if (nvis > cbase[s + 1] - cbase[s]) nvis = cbase[s + 1] - cbase[s];
                for (int g = 0; g < G; ++g) {
                    const float *qr = q + ((size_t)t * Hq + h * G + g) * d;
                    double m = -INFINITY;
                    for (int64_t c = 0; c < nvis; ++c) {
                        const double *kr = kc + ((size_t)(cbase[s] + c) * Hkv + h) * d;
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e) acc += (double)qr[e] * kr[e];
                        p[c] = scale * acc;
                        if (p[c] > m) m = p[c];
                    }
                    double l = 0.0;
                    for (int64_t c = 0; c < nvis; ++c) {
                        p[c] = exp(p[c] - m);
                        l += p[c];
                    }
                    for (int64_t c = 0; c < nvis; ++c) {
                        double w = p[c] / l;
                        int64_t lo = c * stride, hi = c * stride + ks;  /* [lo, hi) */
                        for (int64_t j = lo / bs; j * bs < hi && j <= b; ++j) im[j] += w;
                    }
                }
                memset(taken, 0, (size_t)nbmax);
                int n = 0;
                for (int j = 0; j < init_blocks && n < topk; ++j)
                    if (j <= b && !taken[j]) { taken[j] = 1; out[n++] = j; }
                for (int u = 0; u < local_blocks && n < topk; ++u) {
                    int j = b - u;
                    if (j >= 0 && !taken[j]) { taken[j] = 1; out[n++] = j; }
                }
                while (n < topk) {
                    int best = -1;
                    for (int j = 0; j <= b; ++j)
                        if (!taken[j] && (best < 0 || im[j] > im[best])) best = j;
                    if (best < 0) break;
                    taken[best] = 1;
                    out[n++] = best;
                }
                if (imp) memcpy(imp + (size_t)r * nbmax, im, sizeof(double) * (size_t)nbmax);
            }
        }
        free(p); free(im); free(taken);
    }
    free(kc); free(cbase);
    return bad ? -1 : 0;
}
