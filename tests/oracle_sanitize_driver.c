/* Runs every oracle entry point on small seeded inputs, including empty
 * prefixes, empty lists and bf16 bit patterns, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer sees every code path.
 * Exit status 0 when every call returns 0 and the results are finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/vegas_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* xorshift64*, top 53 bits */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float gauss(void) { return (float)(sqrt(-2.0 * log(unif() + 1e-300)) * cos(6.283185307179586 * unif())); }

static int all_finite(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static int run_case(int dtype, int batch, int hq, int hkv, int d, int gamma, const int* prefixes, int window) {
    const int W = gamma + 1;
    int32_t* cu = calloc((size_t)batch + 1, sizeof(int32_t));
    for (int b = 0; b < batch; ++b) cu[b + 1] = cu[b] + prefixes[b] + W;
    const int64_t total = cu[batch];
    const size_t nq = (size_t)batch * W * hq * d, nkv = (size_t)total * hkv * d;
    const size_t es = dtype == VO_DTYPE_F32 ? 4 : 2;
    unsigned char* q = malloc(nq * es);
    unsigned char* k = malloc(nkv * es);
    unsigned char* v = malloc(nkv * es);
    for (size_t i = 0; i < nq; ++i) {
        float x = gauss();
        if (dtype == VO_DTYPE_F32) memcpy(q + 4 * i, &x, 4);
        else { uint32_t u; memcpy(&u, &x, 4); uint16_t h = (uint16_t)(u >> 16); memcpy(q + 2 * i, &h, 2); }
    }
    for (size_t i = 0; i < nkv; ++i) {
        float x = gauss(), y = gauss();
        if (dtype == VO_DTYPE_F32) { memcpy(k + 4 * i, &x, 4); memcpy(v + 4 * i, &y, 4); }
        else {
            uint32_t u; uint16_t h;
            memcpy(&u, &x, 4); h = (uint16_t)(u >> 16); memcpy(k + 2 * i, &h, 2);
            memcpy(&u, &y, 4); h = (uint16_t)(u >> 16); memcpy(v + 2 * i, &h, 2);
        }
    }
    const double scale = 1.0 / sqrt((double)d);
    double* out = calloc(nq, sizeof(double));
    double* scores = calloc((size_t)hkv * total, sizeof(double));
    int rc = window > 0 ? vo_verify_attn_local(dtype, batch, hq, hkv, d, gamma, scale, q, k, v, cu, total, window,
                                               0u, out, NULL)
                        : vo_verify_attn(dtype, batch, hq, hkv, d, gamma, scale, q, k, v, cu, total,
                                         1u | (1u << gamma), out, scores);
    if (rc || !all_finite(out, nq)) { fprintf(stderr, "verify failed\n"); return 1; }

    int32_t* cuk = calloc((size_t)batch + 1, sizeof(int32_t));
    for (int b = 0; b < batch; ++b) cuk[b + 1] = cuk[b] + prefixes[b] / 3;
    int32_t* idx = calloc((size_t)cuk[batch] + 1, sizeof(int32_t));
    double* theta = calloc((size_t)batch, sizeof(double));
    double* S = calloc((size_t)total, sizeof(double));
    if (window == 0) {
        rc = vo_select_topk(batch, hkv, gamma, scores, cu, total, cuk, idx, theta, S);
        if (rc) { fprintf(stderr, "select failed\n"); return 1; }
    } else {
        rc = vo_streaming_indices(batch, gamma, 2, cu, cuk, idx);
        if (rc) { fprintf(stderr, "streaming failed\n"); return 1; }
    }
    double* dout = calloc((size_t)batch * hq * d, sizeof(double));
    rc = vo_sparse_decode_attn(dtype, batch, hq, hkv, d, scale, q, k, v, cu, idx, cuk, dout);
    if (rc || !all_finite(dout, (size_t)batch * hq * d)) { fprintf(stderr, "decode failed\n"); return 1; }

    free(q); free(k); free(v); free(out); free(scores); free(cu); free(cuk); free(idx); free(theta);
    free(S); free(dout);
    return 0;
}

static int run_accept(int batch, int gamma, int vocab) {
    float* p = malloc(sizeof(float) * (size_t)batch * (gamma + 1) * vocab);
    float* q = malloc(sizeof(float) * ((size_t)batch * gamma * vocab + 1));
    int32_t* draft = malloc(sizeof(int32_t) * ((size_t)batch * gamma + 1));
    float* ua = malloc(sizeof(float) * ((size_t)batch * gamma + 1));
    float* us = malloc(sizeof(float) * (size_t)batch);
    int32_t* na = malloc(sizeof(int32_t) * (size_t)batch);
    int32_t* nt = malloc(sizeof(int32_t) * (size_t)batch);
    for (int r = 0; r < batch * (gamma + 1); ++r) {
        double z = 0; for (int y = 0; y < vocab; ++y) z += (p[(size_t)r * vocab + y] = (float)unif());
        for (int y = 0; y < vocab; ++y) p[(size_t)r * vocab + y] = (float)(p[(size_t)r * vocab + y] / z);
    }
    for (int r = 0; r < batch * gamma; ++r) {
        double z = 0; for (int y = 0; y < vocab; ++y) z += (q[(size_t)r * vocab + y] = (float)unif());
        for (int y = 0; y < vocab; ++y) q[(size_t)r * vocab + y] = (float)(q[(size_t)r * vocab + y] / z);
        draft[r] = (int32_t)(unif() * vocab);
        ua[r] = (float)unif();
    }
    for (int b = 0; b < batch; ++b) us[b] = (float)unif();
    const int rc = vo_spec_accept(batch, gamma, vocab, p, gamma ? q : NULL, gamma ? draft : NULL,
                                  gamma ? ua : NULL, us, na, nt);
    int bad = rc != 0;
    for (int b = 0; b < batch && !bad; ++b) bad = na[b] < 0 || na[b] > gamma || nt[b] < 0 || nt[b] >= vocab;
    free(p); free(q); free(draft); free(ua); free(us); free(na); free(nt);
    if (bad) fprintf(stderr, "accept failed\n");
    return bad;
}

int main(void) {
    const int pre_a[3] = {0, 37, 300};
    const int pre_b[2] = {1, 129};
    const int pre_c[1] = {65};
    int bad = 0;
    bad |= run_case(VO_DTYPE_BF16, 3, 8, 2, 64, 4, pre_a, 0);
    bad |= run_case(VO_DTYPE_F32, 2, 4, 4, 8, 0, pre_b, 0);
    bad |= run_case(VO_DTYPE_F32, 1, 16, 2, 128, 7, pre_c, 0);
    bad |= run_case(VO_DTYPE_BF16, 3, 8, 1, 64, 3, pre_a, 16);
    bad |= run_accept(3, 4, 1000);
    bad |= run_accept(2, 0, 17);
    if (!bad) printf("oracle sanitize driver: ok\n");
    return bad;
}
