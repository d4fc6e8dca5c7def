/* Drives every oracle entry point over small batches (empty events, events
 * at and around num_patches, tie-rich coordinates, kNN lists longer than the
 * event, Lloyd, every pooling variant, the pooling gradient, packing and the
 * random start), each buffer allocated at its exact size, so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer reports any access
 * outside a buffer or any undefined operation in the oracle.  Test
 * infrastructure: built and run by tests/test_oracle_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_sample(const float*, const int64_t*, int64_t, int32_t, const int32_t*, int32_t*,
                  float*, int32_t*, int32_t*);
int oracle_assign(const float*, const int64_t*, int64_t, int32_t, const float*, const int32_t*,
                  int32_t*);
int oracle_tokenize(const float*, const float*, const int64_t*, int64_t, int32_t, int32_t,
                    int32_t, int32_t, int32_t, int32_t, int32_t, const int32_t*, int32_t*, float*,
                    int32_t*, int32_t*, int32_t*, float*, int32_t*);
int oracle_pool_backward(const float*, const int64_t*, int64_t, int32_t, int32_t, int32_t,
                         int32_t, int32_t, int32_t, const int32_t*, const int32_t*,
                         const int32_t*, const float*, const float*, float*);
int oracle_pack(const int32_t*, int64_t, int32_t, int32_t, const float*, float*, int32_t*,
                int32_t*);
int oracle_unpack(const int32_t*, int64_t, int32_t, int32_t, const int32_t*, const float*,
                  float*);
int oracle_random_start(const int64_t*, int64_t, uint64_t, uint64_t, int32_t*);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)
{ /* splitmix64 */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float uniform(float lo, float hi)
{
    return lo + (hi - lo) * (float)((next_u64() >> 40) * (1.0 / 16777216.0));
}

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(3); }
    return p;
}

static int run_case(const int64_t* sizes, int64_t B, int32_t P, int32_t C, int32_t q,
                    int32_t mode, int32_t k, int32_t L, int32_t weighted, int ties)
{
    int64_t* off = xmalloc(sizeof(int64_t) * (size_t)(B + 1));
    off[0] = 0;
    for (int64_t b = 0; b < B; ++b) off[b + 1] = off[b] + sizes[b];
    const int64_t N = off[B];
    float* x = xmalloc(sizeof(float) * (size_t)(4 * N));
    float* f = xmalloc(sizeof(float) * (size_t)(C * N));
    for (int64_t i = 0; i < 4 * N; ++i)
        x[i] = ties ? (float)(int)uniform(0.0f, 3.0f) : uniform(-1.0f, 1.0f);
    for (int64_t i = 0; i < C * N; ++i) f[i] = uniform(-2.0f, 2.0f);
    if (q >= 0)
        for (int64_t i = 0; i < N; ++i) f[i * C + q] = (i % 11 == 0) ? 0.0f : uniform(0.0f, 3.0f);
    int32_t* st = xmalloc(sizeof(int32_t) * (size_t)B);
    if (oracle_random_start(off, B, 7, 3, st)) return 10;
    int32_t* sel = xmalloc(sizeof(int32_t) * (size_t)(B * P));
    float* cen = xmalloc(sizeof(float) * (size_t)(B * P * 4));
    int32_t* tc = xmalloc(sizeof(int32_t) * (size_t)B);
    int32_t* asg = xmalloc(sizeof(int32_t) * (size_t)N);
    int32_t* kn = mode == 1 ? xmalloc(sizeof(int32_t) * (size_t)(B * P * k)) : NULL;
    float* pooled = xmalloc(sizeof(float) * (size_t)(B * P * C));
    int32_t* cnt = xmalloc(sizeof(int32_t) * (size_t)(B * P));
    if (oracle_tokenize(x, f, off, B, C, q, P, mode, k, L, weighted, st, sel, cen, tc, asg, kn,
                        pooled, cnt))
        return 11;
    for (int64_t b = 0; b < B; ++b)
        if (tc[b] != (sizes[b] < P ? sizes[b] : P)) return 12;
    if (oracle_sample(x, off, B, P, NULL, sel, cen, tc, NULL)) return 13;
    if (oracle_assign(x, off, B, P, cen, tc, asg)) return 14;
    float* gp = xmalloc(sizeof(float) * (size_t)(B * P * C));
    for (int64_t i = 0; i < B * P * C; ++i) gp[i] = uniform(-1.0f, 1.0f);
    float* gf = xmalloc(sizeof(float) * (size_t)(C * N));
    if (oracle_pool_backward(f, off, B, C, q, P, mode, mode == 1 ? k : 1, weighted, tc, asg, kn,
                             pooled, gp, gf))
        return 15;
    int64_t T = 0;
    for (int64_t b = 0; b < B; ++b) T += tc[b];
    float* packed = xmalloc(sizeof(float) * (size_t)(T * C));
    int32_t* doc = xmalloc(sizeof(int32_t) * (size_t)T);
    int32_t* cu = xmalloc(sizeof(int32_t) * (size_t)(B + 1));
    if (oracle_pack(tc, B, P, C, pooled, packed, doc, cu)) return 16;
    float* rows = xmalloc(sizeof(float) * (size_t)(B * P * C));
    if (oracle_unpack(tc, B, P, C, cu, packed, rows)) return 17;
    free(off); free(x); free(f); free(st); free(sel); free(cen); free(tc); free(asg); free(kn);
    free(pooled); free(cnt); free(gp); free(gf); free(packed); free(doc); free(cu); free(rows);
    return 0;
}

int main(void)
{
    const int64_t sizes[] = {0, 1, 5, 6, 7, 8, 63, 64, 65, 300, 1000, 0, 2};
    const int64_t B = (int64_t)(sizeof(sizes) / sizeof(sizes[0]));
    const int32_t Ps[] = {1, 7, 64};
    int cases = 0;
    for (int pi = 0; pi < 3; ++pi)
        for (int mode = 0; mode < 2; ++mode)
            for (int L = 0; L <= 2; L += 2)
                for (int w = 0; w < 2; ++w)
                    for (int ties = 0; ties < 2; ++ties) {
                        const int32_t k = mode == 1 ? (ties ? 64 : 16) : 1;
                        const int32_t q = w ? 5 : -1;
                        int rc = run_case(sizes, B, Ps[pi], 6, q, mode, k, L, w, ties);
                        if (rc) {
                            fprintf(stderr, "case P=%d mode=%d L=%d w=%d ties=%d failed: %d\n",
                                    Ps[pi], mode, L, w, ties, rc);
                            return rc;
                        }
                        ++cases;
                    }
    /* an empty batch */
    if (run_case(sizes, 0, 8, 3, -1, 0, 1, 1, 0, 0)) return 20;
    printf("oracle sanitizer driver: %d cases ok\n", cases);
    return 0;
}
