/*
 * fpstok_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, single-threaded CPU implementation of the FPS tokenizer of
 * the Neptune point transformer.  It exists only to decide what the correct
 * answer is.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg
 * of bench.py may load or run it; the GPU library never links it, and the
 * two share no source, header, table or helper.
 *
 * Sources (page title, section):
 *   [PR]  graphnet pull request #923, "Add Neptune point-transformer
 *         backbone": "Summary" (4D (x,y,z,t) cloud, FPS down to at most
 *         num_patches centroids, per-token pooling), "What is added" (small
 *         events keep one token per pulse; Voronoi or kNN pooling; the
 *         function family farthest_point_sampling[_with_assign|_with_knn] and
 *         nearest_assign), the review reply on standardization (time enters
 *         FPS only through differences), the review reply on the no-charge
 *         case (unit charge), and the review reply on the removed precision
 *         argument (FPS is always computed in float32).
 *   [RM]  README of felixyu7/neptune, "Neptune: An Efficient Point
 *         Transformer for Ultrarelativistic Neutrino Events": "Usage"
 *         (coords [N,4] with time in the fourth column, features, per-point
 *         batch ids), "How it works" step 1 (FPS, Voronoi or kNN pooling,
 *         optional charge-weighted Lloyd refinement), "Parameters"
 *         (num_patches, assign_mode, lloyd_iters, k_neighbors).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - squared distance = ((dx*dx + dy*dy) + dz*dz) + dt*dt in float32, each
 *     operation rounded separately (this file must be built with
 *     -ffp-contract=off and without -ffast-math);
 *   - FPS starts at each event's first pulse unless a start index is given;
 *   - argmax ties go to the lowest pulse index, and only pulses not yet
 *     selected compete;
 *   - events with n <= P pass through (token t = pulse t);
 *   - Voronoi ties go to the lowest token slot (selection order);
 *   - kNN lists are ascending in (distance, pulse index), k > n pads with -1;
 *     for a pass-through event the list of token t is [t, -1, ...];
 *   - one Lloyd iteration = charge-weighted mean of each cell accumulated in
 *     float64 in ascending pulse order and rounded to float32 (an empty or
 *     zero-weight cell keeps its centroid), then a fresh nearest-centroid
 *     assignment; pass-through events are skipped;
 *   - pooling = (weighted) mean of every feature column of each token's
 *     members, accumulated in float64, rounded to float32, 0 when the
 *     weight sum is 0;
 *   - indices are event-local int32; slots j >= T are padded with -1 / 0;
 *   - inputs in binary16 or bfloat16 are upcast exactly to float32 first
 *     (every such value is a float32 value) and the float32 path runs on
 *     them: FPS itself stays float32 ([PR] review reply on the removed
 *     precision argument; "What is added": tests in low precision).
 *
 * Layout: coords [N,4] f32 row-major, features [N,C] f32 row-major,
 * offsets [B+1] int64 (CSR, events contiguous), per-event outputs [B,P,...].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with -ffast-math"
#endif

/* Squared 4D distance in float32, fixed axis order, no contraction. */
static float sqdist4(const float* a, const float* c)
{
    float dx = a[0] - c[0];
    float dy = a[1] - c[1];
    float dz = a[2] - c[2];
    float dt = a[3] - c[3];
    float r = dx * dx;
    r = r + dy * dy;
    r = r + dz * dz;
    r = r + dt * dt;
    return r;
}

/* Weight of pulse i: its charge column, or 1 when there is no charge column
 * ([PR] review reply on the no-charge case). */
static double weight_of(const float* f, int32_t C, int32_t charge_col, int64_t i)
{
    if (charge_col < 0) return 1.0;
    return (double)f[i * (int64_t)C + charge_col];
}

/* ------------------------------------------------------------------ FPS -- */

/* Farthest point sampling of one event with the nearest-centroid assignment
 * fused in ([PR] "What is added": farthest_point_sampling_with_assign).
 *   p      : [n,4] the event's pulses
 *   sel    : [P]   output, selected pulse indices in selection order
 *   nearest: [n]   output, slot of the nearest selected pulse (may be NULL)
 * Requires n > P >= 1 and 0 <= start < n. */
static int fps_event(const float* p, int64_t n, int32_t P, int64_t start,
                     int32_t* sel, int32_t* nearest)
{
    float* mind = (float*)malloc((size_t)n * sizeof(float));
    int32_t* near = (int32_t*)malloc((size_t)n * sizeof(int32_t));
    unsigned char* taken = (unsigned char*)calloc((size_t)n, 1);
    if (!mind || !near || !taken) { free(mind); free(near); free(taken); return 1; }
    for (int64_t i = 0; i < n; ++i) { mind[i] = INFINITY; near[i] = 0; }

    int64_t s = start;
    for (int32_t j = 0; j < P; ++j) {
        sel[j] = (int32_t)s;
        taken[s] = 1;
        const float* c = p + 4 * s;
        /* every pulse: distance to the newest centroid; keep the running
         * minimum and the slot that attains it (strict <, so the earliest
         * slot wins a tie) */
        for (int64_t i = 0; i < n; ++i) {
            float d = sqdist4(p + 4 * i, c);
            if (d < mind[i]) { mind[i] = d; near[i] = j; }
        }
        if (j + 1 < P) {
            /* next centroid: the unselected pulse farthest from all chosen
             * so far; strict > keeps the lowest index on ties */
            int64_t best = -1;
            float bestv = 0.0f;
            for (int64_t i = 0; i < n; ++i) {
                if (taken[i]) continue;
                if (best < 0 || mind[i] > bestv) { best = i; bestv = mind[i]; }
            }
            s = best;
        }
    }
    if (nearest) memcpy(nearest, near, (size_t)n * sizeof(int32_t));
    free(mind); free(near); free(taken);
    return 0;
}

/* Batch-level sampling: for each event, FPS (n > P) or pass-through (n <= P).
 *   start_idx   : [B] event-local start pulse, or NULL for 0
 *   centroid_idx: [B,P] int32, -1 padded
 *   centroids   : [B,P,4] f32, 0 padded
 *   token_count : [B] int32, T = min(n, P)
 *   assign      : [N] int32 or NULL (Voronoi slot of each pulse)
 * Returns 0, or 1 on allocation failure, 2 on a bad start index. */
int oracle_sample(const float* coords, const int64_t* offsets, int64_t B, int32_t P,
                  const int32_t* start_idx, int32_t* centroid_idx, float* centroids,
                  int32_t* token_count, int32_t* assign)
{
    for (int64_t b = 0; b < B; ++b) {
        int64_t off = offsets[b];
        int64_t n = offsets[b + 1] - off;
        const float* p = coords + 4 * off;
        int32_t* sel = centroid_idx + b * (int64_t)P;
        float* cen = centroids + b * (int64_t)P * 4;
        int32_t T = (int32_t)(n < P ? n : P);
        token_count[b] = T;
        if (n <= P) {
            /* small events keep one token per pulse ([PR] "What is added") */
            for (int64_t i = 0; i < n; ++i) {
                sel[i] = (int32_t)i;
                memcpy(cen + 4 * i, p + 4 * i, 4 * sizeof(float));
                if (assign) assign[off + i] = (int32_t)i;
            }
        } else {
            int64_t s0 = start_idx ? start_idx[b] : 0;
            if (s0 < 0 || s0 >= n) return 2;
            if (fps_event(p, n, P, s0, sel, assign ? assign + off : NULL)) return 1;
            for (int32_t j = 0; j < P; ++j)
                memcpy(cen + 4 * j, p + 4 * (int64_t)sel[j], 4 * sizeof(float));
        }
        for (int32_t j = T; j < P; ++j) {
            sel[j] = -1;
            memset(cen + 4 * j, 0, 4 * sizeof(float));
        }
    }
    return 0;
}

/* --------------------------------------------------------------- assign -- */

/* Nearest given centroid for every pulse ([PR] "What is added":
 * nearest_assign): argmin over the event's T centroids, lowest slot on ties.
 * Events with T = 0 have no pulses. */
int oracle_assign(const float* coords, const int64_t* offsets, int64_t B, int32_t P,
                  const float* centroids, const int32_t* token_count, int32_t* assign)
{
    for (int64_t b = 0; b < B; ++b) {
        int64_t off = offsets[b];
        int64_t n = offsets[b + 1] - off;
        int32_t T = token_count[b];
        const float* cen = centroids + b * (int64_t)P * 4;
        if (n > 0 && T < 1) return 2;
        for (int64_t i = 0; i < n; ++i) {
            const float* q = coords + 4 * (off + i);
            int32_t best = 0;
            float bd = sqdist4(q, cen);
            for (int32_t j = 1; j < T; ++j) {
                float d = sqdist4(q, cen + 4 * j);
                if (d < bd) { bd = d; best = j; }
            }
            assign[off + i] = best;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ kNN -- */

typedef struct { float d; int32_t i; } dist_idx;

static int cmp_dist_idx(const void* a, const void* b)
{
    const dist_idx* x = (const dist_idx*)a;
    const dist_idx* y = (const dist_idx*)b;
    if (x->d < y->d) return -1;
    if (x->d > y->d) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

/* k nearest pulses of each token's centroid ([PR] "What is added":
 * farthest_point_sampling_with_knn; [RM] "How it works", assign_mode="knn").
 * Lists ascend in (distance, pulse index); k > n pads with -1; a
 * pass-through event's token t gets [t, -1, ...].
 *   knn_idx: [B,P,k] int32 */
int oracle_knn(const float* coords, const int64_t* offsets, int64_t B, int32_t P, int32_t k,
               const float* centroids, const int32_t* token_count, int32_t* knn_idx)
{
    for (int64_t b = 0; b < B; ++b) {
        int64_t off = offsets[b];
        int64_t n = offsets[b + 1] - off;
        int32_t T = token_count[b];
        int32_t* out = knn_idx + b * (int64_t)P * k;
        for (int64_t e = 0; e < (int64_t)P * k; ++e) out[e] = -1;
        if (n <= P) {
            for (int32_t t = 0; t < T; ++t) out[(int64_t)t * k] = t;
            continue;
        }
        dist_idx* buf = (dist_idx*)malloc((size_t)n * sizeof(dist_idx));
        if (!buf) return 1;
        const float* cen = centroids + b * (int64_t)P * 4;
        for (int32_t j = 0; j < T; ++j) {
            for (int64_t i = 0; i < n; ++i) {
                buf[i].d = sqdist4(coords + 4 * (off + i), cen + 4 * j);
                buf[i].i = (int32_t)i;
            }
            qsort(buf, (size_t)n, sizeof(dist_idx), cmp_dist_idx);
            int64_t m = n < k ? n : k;
            for (int64_t e = 0; e < m; ++e) out[(int64_t)j * k + e] = buf[e].i;
        }
        free(buf);
    }
    return 0;
}

/* ---------------------------------------------------------------- Lloyd -- */

/* L rounds of charge-weighted Lloyd refinement ([RM] "How it works": optional
 * charge-weighted Lloyd refinement of the centroids; "Parameters":
 * lloyd_iters).  One round: for every token, c = sum(w p) / sum(w) over the
 * pulses assigned to it, accumulated in float64 in ascending pulse order and
 * rounded to float32 (kept unchanged when the weight sum is 0); then every
 * pulse is re-assigned to its nearest centroid.  Events with n <= P are left
 * untouched.  centroids and assign are read and written in place. */
int oracle_lloyd(const float* coords, const float* features, const int64_t* offsets,
                 int64_t B, int32_t C, int32_t charge_col, int32_t P, int32_t L,
                 float* centroids, const int32_t* token_count, int32_t* assign)
{
    double* acc = (double*)malloc((size_t)P * 5 * sizeof(double));
    if (!acc) return 1;
    for (int64_t b = 0; b < B; ++b) {
        int64_t off = offsets[b];
        int64_t n = offsets[b + 1] - off;
        if (n <= P) continue;
        int32_t T = token_count[b];
        float* cen = centroids + b * (int64_t)P * 4;
        for (int32_t it = 0; it < L; ++it) {
            memset(acc, 0, (size_t)P * 5 * sizeof(double));
            for (int64_t i = 0; i < n; ++i) {
                int32_t j = assign[off + i];
                if (j < 0 || j >= T) { free(acc); return 2; }
                double w = weight_of(features, C, charge_col, off + i);
                const float* q = coords + 4 * (off + i);
                acc[5 * j + 0] += w;
                for (int a = 0; a < 4; ++a) acc[5 * j + 1 + a] += w * (double)q[a];
            }
            for (int32_t j = 0; j < T; ++j) {
                double W = acc[5 * j];
                if (W > 0.0)
                    for (int a = 0; a < 4; ++a) cen[4 * j + a] = (float)(acc[5 * j + 1 + a] / W);
            }
            for (int64_t i = 0; i < n; ++i) {
                const float* q = coords + 4 * (off + i);
                int32_t best = 0;
                float bd = sqdist4(q, cen);
                for (int32_t j = 1; j < T; ++j) {
                    float d = sqdist4(q, cen + 4 * j);
                    if (d < bd) { bd = d; best = j; }
                }
                assign[off + i] = best;
            }
        }
    }
    free(acc);
    return 0;
}

/* ----------------------------------------------------------------- pool -- */

/* Per-token pooling of the pulse features ([PR] "Summary": pools the pulses
 * of each token; [RM] "How it works").  mode 0 (Voronoi): the members of
 * token j are the pulses with assign = j, in ascending order; mode 1 (kNN):
 * the entries != -1 of the token's list, in list order.  Weight: the charge
 * column when weighted != 0, else 1.  pooled[j][c] = sum(w f[c]) / sum(w)
 * accumulated in float64, rounded to float32, 0 when sum(w) = 0.
 *   pooled    : [B,P,C] f32
 *   cell_count: [B,P] int32 member counts (may be NULL) */
int oracle_pool(const float* features, const int64_t* offsets, int64_t B, int32_t C,
                int32_t charge_col, int32_t P, int32_t mode, int32_t k, int32_t weighted,
                const int32_t* token_count, const int32_t* assign, const int32_t* knn_idx,
                float* pooled, int32_t* cell_count)
{
    double* S = (double*)malloc((size_t)P * (size_t)(C + 1) * sizeof(double));
    int32_t* cnt = (int32_t*)malloc((size_t)P * sizeof(int32_t));
    if (!S || !cnt) { free(S); free(cnt); return 1; }
    int32_t wcol = weighted ? charge_col : -1;
    for (int64_t b = 0; b < B; ++b) {
        int64_t off = offsets[b];
        int64_t n = offsets[b + 1] - off;
        int32_t T = token_count[b];
        memset(S, 0, (size_t)P * (size_t)(C + 1) * sizeof(double));
        memset(cnt, 0, (size_t)P * sizeof(int32_t));
        if (mode == 0) {
            for (int64_t i = 0; i < n; ++i) {
                int32_t j = assign[off + i];
                if (j < 0 || j >= T) { free(S); free(cnt); return 2; }
                double w = weight_of(features, C, wcol, off + i);
                double* s = S + (int64_t)j * (C + 1);
                s[0] += w;
                for (int32_t c = 0; c < C; ++c)
                    s[1 + c] += w * (double)features[(off + i) * C + c];
                cnt[j] += 1;
            }
        } else {
            for (int32_t j = 0; j < T; ++j) {
                const int32_t* lst = knn_idx + (b * (int64_t)P + j) * k;
                double* s = S + (int64_t)j * (C + 1);
                for (int32_t e = 0; e < k; ++e) {
                    int32_t i = lst[e];
                    if (i < 0) continue;
                    if (i >= n) { free(S); free(cnt); return 2; }
                    double w = weight_of(features, C, wcol, off + i);
                    s[0] += w;
                    for (int32_t c = 0; c < C; ++c)
                        s[1 + c] += w * (double)features[(off + i) * C + c];
                    cnt[j] += 1;
                }
            }
        }
        float* out = pooled + b * (int64_t)P * C;
        for (int32_t j = 0; j < P; ++j) {
            const double* s = S + (int64_t)j * (C + 1);
            for (int32_t c = 0; c < C; ++c)
                out[(int64_t)j * C + c] = (j < T && s[0] != 0.0) ? (float)(s[1 + c] / s[0]) : 0.0f;
            if (cell_count) cell_count[b * (int64_t)P + j] = j < T ? cnt[j] : 0;
        }
    }
    free(S); free(cnt);
    return 0;
}

/* -------------------------------------------------------- whole pipeline -- */

/* sample -> [Lloyd] -> [kNN] -> pool, the tokenizer as [RM] "How it works"
 * step 1 describes it.  In kNN mode the Voronoi assignment is still computed
 * (Lloyd needs it) and written to `assign`.  `knn_idx` is only written in
 * kNN mode ([B,P,k]). */
int oracle_tokenize(const float* coords, const float* features, const int64_t* offsets,
                    int64_t B, int32_t C, int32_t charge_col, int32_t P, int32_t mode,
                    int32_t k, int32_t L, int32_t weighted, const int32_t* start_idx,
                    int32_t* centroid_idx, float* centroids, int32_t* token_count,
                    int32_t* assign, int32_t* knn_idx, float* pooled, int32_t* cell_count)
{
    int rc = oracle_sample(coords, offsets, B, P, start_idx, centroid_idx, centroids,
                           token_count, assign);
    if (rc) return rc;
    if (L > 0) {
        rc = oracle_lloyd(coords, features, offsets, B, C, charge_col, P, L, centroids,
                          token_count, assign);
        if (rc) return rc;
    }
    if (mode == 1) {
        rc = oracle_knn(coords, offsets, B, P, k, centroids, token_count, knn_idx);
        if (rc) return rc;
    }
    return oracle_pool(features, offsets, B, C, charge_col, P, mode, k, weighted, token_count,
                       assign, knn_idx, pooled, cell_count);
}

/* ------------------------------------------------- token packing (next) -- */

/* Packing of the tokens of a batch into one variable-length sequence for
 * block-diagonal attention ([PR] "What is added": models/utils.py pack /
 * unpack / build_block_mask; the review thread on the packing helper: doc_id
 * is the event index of every packed token and the packed length is the
 * number of tokens).  Event b contributes its first T_b = token_count[b]
 * slots, events in order.
 *   rows      : [B,P,D] per-slot rows (pooled features, centroids, ...)
 *   packed    : [sum T_b, D] the rows of the tokens, event after event
 *   doc_id    : [sum T_b] event of every packed token (may be NULL)
 *   cu_seqlens: [B+1] cu_seqlens[b] = T_0 + ... + T_{b-1}
 * Returns 2 if some T_b is outside [0, P]. */
int oracle_pack(const int32_t* token_count, int64_t B, int32_t P, int32_t D,
                const float* rows, float* packed, int32_t* doc_id, int32_t* cu_seqlens)
{
    int64_t at = 0;
    cu_seqlens[0] = 0;
    for (int64_t b = 0; b < B; ++b) {
        int32_t T = token_count[b];
        if (T < 0 || T > P) return 2;
        for (int32_t j = 0; j < T; ++j) {
            for (int32_t d = 0; d < D; ++d)
                packed[(at + j) * D + d] = rows[(b * P + j) * (int64_t)D + d];
            if (doc_id) doc_id[at + j] = (int32_t)b;
        }
        at += T;
        cu_seqlens[b + 1] = (int32_t)at;
    }
    return 0;
}

/* The inverse: rows[b][j] = packed[cu_seqlens[b] + j] for j < T_b, 0 for
 * T_b <= j < P.  cu_seqlens as oracle_pack writes it. */
int oracle_unpack(const int32_t* token_count, int64_t B, int32_t P, int32_t D,
                  const int32_t* cu_seqlens, const float* packed, float* rows)
{
    for (int64_t b = 0; b < B; ++b) {
        int32_t T = token_count[b];
        if (T < 0 || T > P) return 2;
        for (int32_t j = 0; j < P; ++j)
            for (int32_t d = 0; d < D; ++d)
                rows[(b * P + j) * (int64_t)D + d] =
                    j < T ? packed[((int64_t)cu_seqlens[b] + j) * D + d] : 0.0f;
    }
    return 0;
}

/* ---------------------------------------------- pooling backward (next) -- */

/* Gradient of the pooling (oracle_pool) with respect to the features, given
 * the gradient of the loss with respect to the pooled rows (training runs
 * through the tokenizer: [PR] "Dependencies", time per training step, and
 * "What is added", the gradient tests).  Token j of event b with members
 * M_j (Voronoi: assign = j; kNN: the list entries != -1), weights w_i, weight
 * sum W_j and output m_j = pooled[b][j]:
 *     m_j[c] = sum_{i in M_j} w_i f_i[c] / W_j        (0 when W_j = 0)
 * so, for i in M_j and W_j != 0,
 *     d m_j[c] / d f_i[c'] = [c = c'] w_i / W_j
 *                          + [c' = weight column] (f_i[c] - m_j[c]) / W_j,
 * the second term only when the weights are a feature column (weighted
 * pooling with charge_col >= 0); a token with W_j = 0 has a constant output
 * and contributes nothing.  The mean m_j in that term is the forward's
 * float32 output `pooled`, as an automatic differentiation of the forward
 * would reuse it.  Per pulse the contributions are accumulated in float64 in
 * ascending token order (a pulse is in one Voronoi cell, or in any number of
 * kNN lists); within a token, g_j[c'] * w_i / W_j is formed left to right
 * and the weight-column term as (sum over c ascending of
 * g_j[c] * (f_i[c] - m_j[c])) / W_j.  W_j is the float64 sum of the members'
 * weights in member order (ascending pulse index, or list order), as in
 * oracle_pool.  Result rounded to float32.
 *   grad_pooled  : [B,P,C] f32 (rows j >= T_b are ignored)
 *   pooled       : [B,P,C] f32, the forward output
 *   grad_features: [N,C] f32 out (0 for pulses in no token) */
int oracle_pool_backward(const float* features, const int64_t* offsets, int64_t B, int32_t C,
                         int32_t charge_col, int32_t P, int32_t mode, int32_t k,
                         int32_t weighted, const int32_t* token_count, const int32_t* assign,
                         const int32_t* knn_idx, const float* pooled, const float* grad_pooled,
                         float* grad_features)
{
    int32_t wcol = weighted != 0 ? charge_col : -1;
    int64_t N = offsets[B];
    double* W = (double*)malloc((size_t)(P > 0 ? P : 1) * sizeof(double));
    double* G = (double*)malloc((size_t)(N > 0 ? N : 1) * (size_t)C * sizeof(double));
    if (!W || !G) { free(W); free(G); return 1; }
    memset(G, 0, (size_t)(N > 0 ? N : 1) * (size_t)C * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        int64_t off = offsets[b];
        int64_t n = offsets[b + 1] - off;
        int32_t T = token_count[b];
        if (T < 0 || T > P) { free(W); free(G); return 2; }
        /* weight sums, in member order */
        for (int32_t j = 0; j < P; ++j) W[j] = 0.0;
        if (mode == 0) {
            for (int64_t i = 0; i < n; ++i) {
                int32_t j = assign[off + i];
                if (j < 0 || j >= T) { free(W); free(G); return 2; }
                W[j] += weight_of(features, C, wcol, off + i);
            }
        } else {
            for (int32_t j = 0; j < T; ++j)
                for (int32_t e = 0; e < k; ++e) {
                    int32_t i = knn_idx[(b * (int64_t)P + j) * k + e];
                    if (i < 0) continue;
                    if (i >= n) { free(W); free(G); return 2; }
                    W[j] += weight_of(features, C, wcol, off + i);
                }
        }
        /* contributions of token j to its member i, tokens in ascending order */
        for (int32_t j = 0; j < T; ++j) {
            if (W[j] == 0.0) continue;
            const float* g = grad_pooled + (b * (int64_t)P + j) * C;
            const float* m = pooled + (b * (int64_t)P + j) * C;
            int64_t cnt = mode == 0 ? n : k;
            for (int64_t e = 0; e < cnt; ++e) {
                int64_t i;
                if (mode == 0) {
                    if (assign[off + e] != j) continue;
                    i = e;
                } else {
                    int32_t q = knn_idx[(b * (int64_t)P + j) * k + e];
                    if (q < 0) continue;
                    i = q;
                }
                const float* f = features + (off + i) * (int64_t)C;
                double w = weight_of(features, C, wcol, off + i);
                double* gi = G + (off + i) * (int64_t)C;
                for (int32_t c = 0; c < C; ++c) gi[c] += (double)g[c] * w / W[j];
                if (wcol >= 0) {
                    double s = 0.0;
                    for (int32_t c = 0; c < C; ++c) s += (double)g[c] * ((double)f[c] - (double)m[c]);
                    gi[wcol] += s / W[j];
                }
            }
        }
    }
    for (int64_t q = 0; q < N * (int64_t)C; ++q) grad_features[q] = (float)G[q];
    free(W); free(G);
    return 0;
}

/* ----------------------------------------------- random FPS start (next) -- */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): ten rounds
 * of two 32x32->64-bit multiplications (multipliers 0xD2511F53 and
 * 0xCD9E8D57) mixed with the key, the key advanced by the Weyl constants
 * 0x9E3779B9 and 0xBB67AE85 between rounds. */
static void philox4x32_10(const uint32_t in[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Exposed for the generator's known-answer tests. */
void oracle_philox4x32_10(const uint32_t* in, const uint32_t* key, uint32_t* out)
{
    philox4x32_10(in, key, out);
}

/* A random FPS start per event ([PR] review thread on the FPS arguments:
 * start_idx, random_start, generator; the pages do not say how the start is
 * drawn).  Event b draws word 0 of Philox4x32-10 at counter (b low, b high,
 * step low, step high) with key (seed low, seed high) and maps it to
 * floor(u * n_b / 2^32), a pulse index in [0, n_b); an empty event gets 0.
 *   start_idx: [B] int32 out */
int oracle_random_start(const int64_t* offsets, int64_t B, uint64_t seed, uint64_t step,
                        int32_t* start_idx)
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int64_t b = 0; b < B; ++b) {
        int64_t n = offsets[b + 1] - offsets[b];
        uint32_t in[4] = {(uint32_t)b, (uint32_t)((uint64_t)b >> 32), (uint32_t)step,
                          (uint32_t)(step >> 32)};
        uint32_t out[4];
        philox4x32_10(in, key, out);
        start_idx[b] = n > 0 ? (int32_t)(((uint64_t)out[0] * (uint64_t)n) >> 32) : 0;
    }
    return 0;
}

/* ------------------------------------------ low-precision inputs (next) -- */

/* IEEE 754 binary16 to binary32, from the format's definition: sign bit,
 * 5-bit exponent biased by 15, 10-bit fraction.  Exponent 0 holds zero and
 * the subnormals fraction * 2^-24; exponent 31 holds the infinities (fraction
 * 0) and NaNs (the fraction kept as the top of the binary32 fraction); every
 * other exponent e gives (1024 + fraction) * 2^(e - 25).  Each value is
 * exactly representable in binary32, and ldexpf of an integer below 2^11 is
 * exact, so nothing is rounded. */
static float f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1F;
    const int m = h & 0x3FF;
    float v;
    if (e == 0) {
        v = ldexpf((float)m, -24);
    } else if (e == 31) {
        uint32_t bits = ((uint32_t)sign << 31) | 0x7F800000u | ((uint32_t)m << 13);
        memcpy(&v, &bits, sizeof v);
        return v;
    } else {
        v = ldexpf((float)(1024 + m), e - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 to binary32: bfloat16 is defined as the upper 16 bits of a
 * binary32 (same sign and 8-bit exponent, 7 of the 23 fraction bits), so
 * the value is the binary32 whose low 16 bits are zero. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float v;
    memcpy(&v, &bits, sizeof v);
    return v;
}

/* dst[i] = the float32 value of the 16-bit src[i]; dtype 1 = binary16,
 * 2 = bfloat16.  Returns 2 for another dtype. */
int oracle_upcast(const uint16_t* src, int64_t count, int32_t dtype, float* dst)
{
    if (dtype != 1 && dtype != 2) return 2;
    for (int64_t i = 0; i < count; ++i)
        dst[i] = dtype == 1 ? f16_to_f32(src[i]) : bf16_to_f32(src[i]);
    return 0;
}
