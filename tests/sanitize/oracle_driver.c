/*
 * Test driver for the sanitizer build of oracle/oracle.c (TEST
 * INFRASTRUCTURE): runs every step function on small inputs that reach its
 * edge cases (an empty batch, k = 1, k = E, ties, -0, -inf logits,
 * group-limited routing, empty experts, dropped choices, bf16 and fp32
 * rows) and prints a checksum line per call, so that the sanitized and the
 * plain build can be compared line by line.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_route(const float*, int, int, int, int, int, int32_t*, double*);
int orc_coact(const int32_t*, int, int, int, int64_t*);
int orc_layout(const int32_t*, int, int, int, const int32_t*, int, uint32_t*, int32_t*,
               int32_t*, int32_t*, int32_t*, int32_t*);
int orc_dispatch_rows(const void*, int, int, int, const int32_t*, int, void*);
int orc_ffn_rows(const void*, int, int, int, int, const int32_t*, const int32_t*, int,
                 const void*, const void*, const void*, double*, double*);
int orc_combine(const double*, int, const int32_t*, const double*, int, int, int, double*);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
static float uniform(void) { return (float)(next_u32() >> 8) / 16777216.0f * 4.0f - 2.0f; }

static double sum_d(const double* a, size_t n)
{
    double s = 0.0;
    for (size_t i = 0; i < n; ++i) s += a[i] * (double)(1 + i % 7);
    return s;
}
static long long sum_i(const int32_t* a, size_t n)
{
    long long s = 0;
    for (size_t i = 0; i < n; ++i) s += (long long)a[i] * (long long)(1 + i % 5);
    return s;
}

static int run_case(int T, int E, int k, int ng, int tg, int G, int d, int F, int bf16)
{
    size_t TE = (size_t)T * E, Tk = (size_t)T * k;
    float* logits = malloc(sizeof(float) * (TE ? TE : 1));
    for (size_t i = 0; i < TE; ++i) {
        logits[i] = uniform();
        if (i % 5 == 0) logits[i] = roundf(logits[i]);   /* ties */
        if (i % 23 == 0) logits[i] = -0.0f;
    }
    /* -inf masks that leave every group at least E/ng - 1 finite logits */
    for (int t = 2; t < T; t += 5) logits[(size_t)t * E + (t % (E / ng))] = -INFINITY;
    int32_t* idx = malloc(sizeof(int32_t) * (Tk ? Tk : 1));
    double* gates = malloc(sizeof(double) * (Tk ? Tk : 1));
    int rc = orc_route(logits, T, E, k, ng, tg, idx, gates);
    printf("route rc=%d idx=%lld gates=%.17g\n", rc, sum_i(idx, Tk), sum_d(gates, Tk));
    if (rc) return 1;

    int64_t* co = malloc(sizeof(int64_t) * (size_t)E * E);
    rc = orc_coact(idx, T, E, k, co);
    long long cs = 0;
    for (size_t i = 0; i < (size_t)E * E; ++i) cs += co[i] * (long long)(1 + i % 3);
    printf("coact rc=%d sum=%lld\n", rc, cs);

    int32_t* place = malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e) place[e] = (e * 7) % G;
    uint32_t* rm = malloc(sizeof(uint32_t) * (size_t)(T ? T : 1));
    int32_t* ro = malloc(sizeof(int32_t) * (size_t)(G + 1));
    int32_t* dt = malloc(sizeof(int32_t) * (Tk ? Tk : 1));
    int32_t* eo = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* pr = malloc(sizeof(int32_t) * (Tk ? Tk : 1));
    int32_t* so = malloc(sizeof(int32_t) * (Tk ? Tk : 1));
    rc = orc_layout(idx, T, E, k, place, G, rm, ro, dt, eo, pr, so);
    int R = ro[G];
    printf("layout rc=%d R=%d rows=%lld slots=%lld\n", rc, R, sum_i(dt, (size_t)R),
           sum_i(pr, Tk) + 3 * sum_i(so, Tk) + sum_i(eo, (size_t)E + 1));

    size_t eb = bf16 ? 2 : 4;
    unsigned char* x = malloc(eb * (size_t)(T ? T : 1) * d);
    for (size_t i = 0; i < (size_t)T * d; ++i) {
        float v = uniform();
        if (bf16) {
            uint32_t b;
            memcpy(&b, &v, 4);
            uint16_t h = (uint16_t)(b >> 16);
            memcpy(x + 2 * i, &h, 2);
        } else {
            memcpy(x + 4 * i, &v, 4);
        }
    }
    unsigned char* xd = malloc(eb * (size_t)(R ? R : 1) * d);
    rc = orc_dispatch_rows(x, T, d, (int)eb, dt, R, xd);
    printf("dispatch rc=%d\n", rc);

    size_t wsz = (size_t)E * F * d;
    unsigned char* wg = malloc(eb * wsz);
    unsigned char* wu = malloc(eb * wsz);
    unsigned char* wd = malloc(eb * wsz);
    for (size_t i = 0; i < wsz; ++i) {
        float v[3] = {uniform() / 8, uniform() / 8, uniform() / 8};
        unsigned char* w[3] = {wg, wu, wd};
        for (int q = 0; q < 3; ++q) {
            if (bf16) {
                uint32_t b;
                memcpy(&b, &v[q], 4);
                uint16_t h = (uint16_t)(b >> 16);
                memcpy(w[q] + 2 * i, &h, 2);
            } else {
                memcpy(w[q] + 4 * i, &v[q], 4);
            }
        }
    }
    int32_t* sexp = malloc(sizeof(int32_t) * (Tk ? Tk : 1));
    for (int e = 0; e < E; ++e)
        for (int s = eo[e]; s < eo[e + 1]; ++s) sexp[s] = e;
    double* y = malloc(sizeof(double) * (Tk ? Tk : 1) * d);
    double* h = malloc(sizeof(double) * (Tk ? Tk : 1) * F);
    rc = orc_ffn_rows(xd, bf16, d, F, (int)Tk, pr, sexp, E, wg, wu, wd, y, h);
    printf("ffn rc=%d y=%.17g h=%.17g\n", rc, sum_d(y, Tk * d), sum_d(h, Tk * F));

    /* drop every fifth choice */
    for (size_t i = 0; i < Tk; i += 5) so[i] = -1;
    double* out = malloc(sizeof(double) * (size_t)(T ? T : 1) * d);
    rc = orc_combine(y, (int)Tk, so, gates, T, k, d, out);
    printf("combine rc=%d out=%.17g\n", rc, sum_d(out, (size_t)T * d));

    free(logits); free(idx); free(gates); free(co); free(place); free(rm); free(ro); free(dt);
    free(eo); free(pr); free(so); free(x); free(xd); free(wg); free(wu); free(wd); free(sexp);
    free(y); free(h); free(out);
    return 0;
}

int main(void)
{
    int bad = 0;
    bad |= run_case(37, 8, 2, 1, 1, 4, 16, 24, 1);
    bad |= run_case(20, 8, 8, 1, 1, 2, 8, 8, 0);    /* k = E */
    bad |= run_case(33, 8, 1, 1, 1, 3, 8, 16, 1);   /* k = 1, G does not divide E */
    bad |= run_case(41, 16, 3, 4, 2, 4, 8, 8, 1);   /* group-limited */
    bad |= run_case(5, 64, 2, 1, 1, 32, 8, 8, 0);   /* mostly empty experts, G = 32 */
    bad |= run_case(0, 8, 2, 1, 1, 4, 8, 8, 1);     /* empty batch */
    return bad;
}
