/*
 * TEST INFRASTRUCTURE -- float64 CPU oracle for the fused full-vocabulary binary cross-entropy.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may build, load or call this file.
 * It shares no code, header or constant with the GPU library and is deliberately plain and slow: every
 * logit z is formed as an explicit dot product, in float64, with d ascending, and nothing is blocked,
 * fused or reordered beyond what the definitions below state.
 *
 * What it computes ("Cut Binary Cross Entropy", Li, Ning, Hammad):
 *   - Section III-A, Eq. (1)-(2): per logit x and target y in {0,1}, the BCE loss in its stable form
 *       L(x, y) = max(x, 0) + log(1 + exp(-|x|)) - y * x .
 *   - Section III-A, Eq. (3): per position, the sum over all V items, divided by V; then (Section III-B, the
 *     paragraph after Eq. (4)) averaged over positions with padding positions left out. Together:
 *       loss = 1 / (R_v * V) * sum_{valid rows r} sum_{v < V} L(z_rv, y_rv),  z_rv = H[r] . E[v].
 *   - Section III-B, Eq. (4): dL/dz_rv = s * (sigma(z_rv) - y_rv) with s = 1 / (R_v * V), hence
 *       dH[r] = g * s * sum_v (sigma(z_rv) - y_rv) E[v]   (valid rows; masked rows get 0),
 *       dE[v] = g * s * sum_{valid r} (sigma(z_rv) - y_rv) H[r],
 *     where g is the upstream cotangent of the scalar loss (the custom-VJP input).
 *
 * Readings where the paper is silent (each is listed in the design notes):
 *   - targets are given per row as a list of ids; y_rv = 1 iff v appears in row r's list (a repeated id
 *     counts once, since y is binary in Section III-A);
 *   - the per-position `weights` of the paper's API: a row mask (0 = padding, whose positives are ignored)
 *     and, optionally, a weight w_r per row (1 when none is given). The average over positions becomes the
 *     weighted average: with W = sum of w_r over valid rows and s = 1 / (W * V),
 *       loss  = s * sum_{valid r} w_r sum_v L(z_rv, y_rv),
 *       dH[r] = g * s * w_r * sum_v (sigma(z_rv) - y_rv) E[v],
 *       dE[v] = g * s * sum_{valid r} w_r (sigma(z_rv) - y_rv) H[r];
 *     unit weights give the plain average above (W = R_v);
 *   - W = 0 (every row masked, or all weights 0) gives loss 0 and zero gradients;
 *   - row_loss[r] is the unnormalised, unweighted sum_v L(z_rv, y_rv) of a valid row and 0 for a masked row.
 *
 * Full-vocabulary top-k (Section III-E evaluation): per valid row, the k items with the largest logits, ordered
 * by logit (descending) and, among equal logits, by item id (ascending); Hit@k counts a row as a hit when at
 * least one of its positives is among them.
 *
 * Cut Metrics (Section III-D): per position, the confusion counts TP, FP, FN, TN over the V items, computed
 * from the same logits without materialising them. The section names no threshold; the plain reading used
 * here is "predict positive iff sigma(z) > 1/2", i.e. iff z > 0 (z = 0 is a negative prediction). Masked rows
 * get all-zero counts.
 *
 * Inputs H and E are read either as IEEE float32 or as bfloat16 (dtype 0 / 1), each element converted
 * exactly to double before use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_BAD_SHAPE 1
#define OR_BAD_IDS 2
#define OR_NOMEM 3

/* Planted mistakes: compiled in only for the tests that prove the pins catch them. */
#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

static double load_elem(const void *p, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float *)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16; /* bfloat16 = top half of a float32 */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double bf16_bits_to_double(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16; /* bfloat16 = top half of a float32 */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* z = sum_d H[r][d] * E[v][d], d ascending (one loop per element type; the same products and additions). */
static double dot_rv(const void *H, const void *E, int dtype, int64_t r, int64_t v, int D) {
    double z = 0.0;
    if (dtype == 0) {
        const float *h = (const float *)H + (size_t)r * D, *e = (const float *)E + (size_t)v * D;
        for (int d = 0; d < D; ++d) z += (double)h[d] * (double)e[d];
    } else {
        const uint16_t *h = (const uint16_t *)H + (size_t)r * D, *e = (const uint16_t *)E + (size_t)v * D;
        for (int d = 0; d < D; ++d) z += bf16_bits_to_double(h[d]) * bf16_bits_to_double(e[d]);
    }
    return z;
}

/* Eq. (2): L(x, 0) = max(x, 0) + log(1 + exp(-|x|)). */
static double softplus(double x) {
#if ORACLE_PLANT == 5
    return log1p(exp(-fabs(x))); /* planted: drops max(x, 0) */
#else
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
#endif
}

/* sigma(x), evaluated without overflow on either side. */
static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* Weight of row r: 0 for a masked row, else row_weight[r] (1 without weights). */
static double row_w(const uint8_t *row_mask, const double *row_weight, int64_t r) {
    if (!row_mask[r]) return 0.0;
    return row_weight ? row_weight[r] : 1.0;
}

/* s = 1 / (W * V) with W the summed weight of the valid rows (rows in ascending order); 0 when W = 0. */
static double norm_scale(int64_t R, int64_t V, const uint8_t *row_mask, const double *row_weight) {
    double W = 0.0;
    for (int64_t r = 0; r < R; ++r) {
#if ORACLE_PLANT == 6
        W += row_mask[r] ? 1.0 : 0.0; /* planted: the normaliser ignores the weights */
#else
        W += row_w(row_mask, row_weight, r);
#endif
    }
#if ORACLE_PLANT == 2
    W = (double)R; /* planted: padding rows counted in the average */
#endif
    return W != 0.0 ? 1.0 / (W * (double)V) : 0.0;
}

/* Check CSR consistency and id range; count valid rows. */
static int check_inputs(int64_t R, int64_t V, int D, const int32_t *row_offsets, const int32_t *item_ids,
                        const uint8_t *row_mask, int64_t *n_valid) {
    if (R < 0 || V < 1 || D < 1) return OR_BAD_SHAPE;
    if (row_offsets[0] != 0) return OR_BAD_IDS;
    int64_t rv = 0;
    for (int64_t r = 0; r < R; ++r) {
        if (row_offsets[r + 1] < row_offsets[r]) return OR_BAD_IDS;
        for (int64_t p = row_offsets[r]; p < row_offsets[r + 1]; ++p)
            if (item_ids[p] < 0 || item_ids[p] >= V) return OR_BAD_IDS;
        if (row_mask[r]) ++rv;
    }
    *n_valid = rv;
    return OR_OK;
}

/* y_rv for one row: mark the row's ids in a V-sized byte map (repeated ids collapse). */
static void mark_row(const int32_t *row_offsets, const int32_t *item_ids, int64_t r, uint8_t *ymap, int on) {
    for (int64_t p = row_offsets[r]; p < row_offsets[r + 1]; ++p) ymap[item_ids[p]] = (uint8_t)on;
}

static int cmp_i32(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Is v among row r's ids? `sorted_ids` holds each row's ids sorted (same CSR offsets). */
static int row_has(const int32_t *row_offsets, const int32_t *sorted_ids, int64_t r, int32_t v) {
    int64_t lo = row_offsets[r], hi = row_offsets[r + 1];
    while (lo < hi) {
        int64_t mid = (lo + hi) / 2;
        if (sorted_ids[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo < row_offsets[r + 1] && sorted_ids[lo] == v;
}

static int32_t *sorted_copy(int64_t R, const int32_t *row_offsets, const int32_t *item_ids) {
    int64_t nnz = row_offsets[R];
    int32_t *s = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    if (!s) return NULL;
    if (nnz) memcpy(s, item_ids, sizeof(int32_t) * (size_t)nnz);
    for (int64_t r = 0; r < R; ++r)
        qsort(s + row_offsets[r], (size_t)(row_offsets[r + 1] - row_offsets[r]), sizeof(int32_t), cmp_i32);
    return s;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Row side: for each requested row (n_rows entries of `rows`; all R rows when rows == NULL) compute
 * row_loss[i] = sum_v L(z, y) (0 for a masked row) and, when dH != NULL,
 * dH[i][:] = g*s*w_r*sum_v (sigma-y) E[v] (0 for a masked row). s uses the weight of all valid rows.
 */
int oracle_rows(int64_t R, int64_t V, int D, int dtype, const void *H, const void *E,
                const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask,
                const double *row_weight, double g, int64_t n_rows, const int64_t *rows, double *row_loss,
                double *dH) {
    int64_t rv;
    int st = check_inputs(R, V, D, row_offsets, item_ids, row_mask, &rv);
    if (st) return st;
    if (!rows) n_rows = R;
    const double s = norm_scale(R, V, row_mask, row_weight);
    int err = 0;
#pragma omp parallel
    {
        uint8_t *ymap = (uint8_t *)calloc((size_t)V, 1);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!ymap || !acc) {
#pragma omp atomic write
            err = OR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!ymap || !acc) continue;
            int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= R) {
#pragma omp atomic write
                err = OR_BAD_SHAPE;
                continue;
            }
            if (!row_mask[r]) {
                row_loss[i] = 0.0;
                if (dH) for (int d = 0; d < D; ++d) dH[(size_t)i * D + d] = 0.0;
                continue;
            }
            mark_row(row_offsets, item_ids, r, ymap, 1);
            double lsum = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                double z = dot_rv(H, E, dtype, r, v, D);
                double y = ymap[v] ? 1.0 : 0.0;
#if ORACLE_PLANT == 1
                lsum += softplus(z); /* planted: sparse target correction dropped */
#else
                lsum += softplus(z) - y * z;
#endif
                if (dH) {
#if ORACLE_PLANT == 3
                    double gz = y - sigmoid(z); /* planted: sign of the logit gradient flipped */
#else
                    double gz = sigmoid(z) - y;
#endif
                    for (int d = 0; d < D; ++d) acc[d] += gz * load_elem(E, dtype, (size_t)v * D + d);
                }
            }
            mark_row(row_offsets, item_ids, r, ymap, 0);
            row_loss[i] = lsum;
            if (dH) {
                const double w = row_w(row_mask, row_weight, r);
                for (int d = 0; d < D; ++d) dH[(size_t)i * D + d] = g * s * w * acc[d];
            }
        }
        free(ymap);
        free(acc);
    }
    return err;
}

/* Item side: dE[i][:] = g*s*sum_{valid r} w_r (sigma(z_r,v) - y_r,v) H[r] for each requested item (all V
 * when items == NULL). */
int oracle_items(int64_t R, int64_t V, int D, int dtype, const void *H, const void *E,
                 const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask,
                 const double *row_weight, double g, int64_t n_items, const int64_t *items, double *dE) {
    int64_t rv;
    int st = check_inputs(R, V, D, row_offsets, item_ids, row_mask, &rv);
    if (st) return st;
    if (!items) n_items = V;
    const double s = norm_scale(R, V, row_mask, row_weight);
    int32_t *sorted = sorted_copy(R, row_offsets, item_ids);
    if (!sorted) return OR_NOMEM;
    int err = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!acc) {
#pragma omp atomic write
            err = OR_NOMEM;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n_items; ++i) {
            if (!acc) continue;
            int64_t v = items ? items[i] : i;
            if (v < 0 || v >= V) {
#pragma omp atomic write
                err = OR_BAD_SHAPE;
                continue;
            }
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t r = 0; r < R; ++r) {
                if (!row_mask[r]) continue;
                double z = dot_rv(H, E, dtype, r, v, D);
                double y = row_has(row_offsets, sorted, r, (int32_t)v) ? 1.0 : 0.0;
#if ORACLE_PLANT == 7
                double gz = sigmoid(z) - y; /* planted: the row weight left out of dE */
#else
                double gz = row_w(row_mask, row_weight, r) * (sigmoid(z) - y);
#endif
#if ORACLE_PLANT == 4
                /* planted: transposed operand -- uses E[v] where H[r] belongs */
                for (int d = 0; d < D; ++d) acc[d] += gz * load_elem(E, dtype, (size_t)v * D + d);
#else
                for (int d = 0; d < D; ++d) acc[d] += gz * load_elem(H, dtype, (size_t)r * D + d);
#endif
            }
            for (int d = 0; d < D; ++d) dE[(size_t)i * D + d] = g * s * acc[d];
        }
        free(acc);
    }
    free(sorted);
    return err;
}

/* Whole problem: loss = s * sum of weighted valid row losses in ascending row order, plus optional
 * row_loss [R], dH [R][D] and dE [V][D]. */
int oracle_full(int64_t R, int64_t V, int D, int dtype, const void *H, const void *E,
                const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask,
                const double *row_weight, double g, double *loss, double *row_loss, double *dH, double *dE) {
    int64_t rv;
    int st = check_inputs(R, V, D, row_offsets, item_ids, row_mask, &rv);
    if (st) return st;
    double *rl = row_loss ? row_loss : (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    if (!rl) return OR_NOMEM;
    st = oracle_rows(R, V, D, dtype, H, E, row_offsets, item_ids, row_mask, row_weight, g, R, NULL, rl, dH);
    if (!st && dE)
        st = oracle_items(R, V, D, dtype, H, E, row_offsets, item_ids, row_mask, row_weight, g, V, NULL, dE);
    if (!st) {
        const double s = norm_scale(R, V, row_mask, row_weight);
        double tot = 0.0;
        for (int64_t r = 0; r < R; ++r) tot += row_w(row_mask, row_weight, r) * rl[r];
        *loss = s * tot;
    }
    if (!row_loss) free(rl);
    return st;
}

/*
 * Cut Metrics (Section III-D) for each requested row (all R when rows == NULL): out[i][0..4] =
 * TP, FP, FN, TN with the prediction "z > 0", and the number of items with |z| <= eps (logits whose sign a
 * lower-precision evaluation may decide differently). Masked rows get zeros.
 */
int oracle_metrics(int64_t R, int64_t V, int D, int dtype, const void *H, const void *E,
                   const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask, double eps,
                   int64_t n_rows, const int64_t *rows, int64_t *out) {
    int64_t rv;
    int st = check_inputs(R, V, D, row_offsets, item_ids, row_mask, &rv);
    if (st) return st;
    if (!rows) n_rows = R;
    int err = 0;
#pragma omp parallel
    {
        uint8_t *ymap = (uint8_t *)calloc((size_t)V, 1);
        if (!ymap) {
#pragma omp atomic write
            err = OR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!ymap) continue;
            int64_t r = rows ? rows[i] : i;
            int64_t *o = out + (size_t)i * 5;
            for (int q = 0; q < 5; ++q) o[q] = 0;
            if (r < 0 || r >= R) {
#pragma omp atomic write
                err = OR_BAD_SHAPE;
                continue;
            }
            if (!row_mask[r]) continue;
            mark_row(row_offsets, item_ids, r, ymap, 1);
            for (int64_t v = 0; v < V; ++v) {
                double z = dot_rv(H, E, dtype, r, v, D);
#if ORACLE_PLANT == 8
                int pred = z >= 0.0; /* planted: a zero logit predicted positive */
#else
                int pred = z > 0.0;
#endif
                int y = ymap[v] != 0;
                if (pred && y) ++o[0];
                else if (pred && !y) ++o[1];
                else if (!pred && y) ++o[2];
                else ++o[3];
                if (fabs(z) <= eps) ++o[4];
            }
            mark_row(row_offsets, item_ids, r, ymap, 0);
        }
        free(ymap);
    }
    return err;
}

/* Does (za, va) rank before (zb, vb): larger logit first, smaller item id among equal logits. */
static int ranks_before(double za, int64_t va, double zb, int64_t vb) {
#if ORACLE_PLANT == 9
    return za > zb || (za == zb && va > vb); /* planted: ties broken towards the larger id */
#else
    return za > zb || (za == zb && va < vb);
#endif
}

/*
 * Full-vocabulary top-k for each requested row (all R when rows == NULL): ids[i][0..k) and vals[i][0..k) hold
 * the k best items of row r in rank order (see ranks_before) and their float64 logits; hits[i] (when hits !=
 * NULL) counts how many of them are among the row's positives. Masked rows get ids -1, vals -inf, hits 0.
 * Requires 1 <= k <= V.
 */
int oracle_topk(int64_t R, int64_t V, int D, int dtype, const void *H, const void *E,
                const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask, int k,
                int64_t n_rows, const int64_t *rows, int64_t *ids, double *vals, int64_t *hits) {
    int64_t rv;
    int st = check_inputs(R, V, D, row_offsets, item_ids, row_mask, &rv);
    if (st) return st;
    if (k < 1 || k > V) return OR_BAD_SHAPE;
    if (!rows) n_rows = R;
    int err = 0;
#pragma omp parallel
    {
        uint8_t *ymap = (uint8_t *)calloc((size_t)V, 1);
        if (!ymap) {
#pragma omp atomic write
            err = OR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!ymap) continue;
            int64_t r = rows ? rows[i] : i;
            int64_t *id = ids + (size_t)i * k;
            double *va = vals + (size_t)i * k;
            for (int q = 0; q < k; ++q) {
                id[q] = -1;
                va[q] = -INFINITY;
            }
            if (hits) hits[i] = 0;
            if (r < 0 || r >= R) {
#pragma omp atomic write
                err = OR_BAD_SHAPE;
                continue;
            }
            if (!row_mask[r]) continue;
            /* insertion into a sorted list of the k best so far */
            int64_t filled = 0;
            for (int64_t v = 0; v < V; ++v) {
                double z = dot_rv(H, E, dtype, r, v, D);
                if (filled == k && !ranks_before(z, v, va[k - 1], id[k - 1])) continue;
                int64_t q = filled < k ? filled++ : k - 1;
                while (q > 0 && ranks_before(z, v, va[q - 1], id[q - 1])) {
                    va[q] = va[q - 1];
                    id[q] = id[q - 1];
                    --q;
                }
                va[q] = z;
                id[q] = v;
            }
            if (hits) {
                mark_row(row_offsets, item_ids, r, ymap, 1);
                for (int q = 0; q < k; ++q) hits[i] += ymap[id[q]] ? 1 : 0;
                mark_row(row_offsets, item_ids, r, ymap, 0);
            }
        }
        free(ymap);
    }
    return err;
}
